/* A plain C99 client of include/spkv.h (no C++, no Python): drives a
 * host-only handle through the append -> evict -> plan steps of a stream and
 * prints, per frame, the plan, the free list and the stats, then the codes
 * of a few calls whose result the contract fixes.  tests/test_c_client.py
 * builds it with gcc, runs it and checks the output.
 *
 * usage: c_abi_client NB H D PS P NS S W R MTF FRAMES
 *        c_abi_client script NB H D PS P NS S W R MTF < commands
 *
 * Script mode reads one command per line and applies it to block 0 of a
 * host-only handle, printing "<command> <code>" for each:
 *   a          append_frame_in_run        A      append_frame
 *   e C M      evict_frames with cross_frame_special C and camera_only M
 *   d E        set_defer_eviction(E)      x      execute_deferred_eviction
 *   r          rollback_last_frame
 *   p          plan, then the plan's table, last_page_len, special runs, the
 *              block's special runs and its free list on the same line
 *   c          the codes of run, run_own, run_noalloc (host-only: all checks,
 *              then UNSUPPORTED) and set_num_splits(3) and (-1)
 *   R          reset                      s      get_cache_stats, printed */
#include <stdio.h>
#include <stdlib.h>

#include "spkv.h"

#define CAP 4096

static void print_list(const char* tag, const int32_t* v, int32_t n) {
  int32_t i;
  printf(" %s", tag);
  for (i = 0; i < n; ++i) printf(" %d", (int)v[i]);
}

static int script(spkv_config* c) {
  static int32_t table[CAP], runs[3 * CAP], scale[CAP], live[CAP], free_list[CAP];
  int32_t n_pages, n_patch, lpl, n_runs, n_scale, n_live, n_free;
  int64_t nsf;
  spkv_handle* h = NULL;
  char cmd[8];
  int a1, a2, rc;
  const int32_t nq = c->num_special_tokens + c->patch_tokens;
  rc = spkv_create(c, NULL, NULL, 0, &h);
  printf("create %d\n", rc);
  if (rc != SPKV_OK) return 1;
  while (scanf("%7s", cmd) == 1) {
    switch (cmd[0]) {
      case 'a': printf("a %d\n", spkv_append_frame_in_run(h, 0, NULL, NULL, NULL)); break;
      case 'A': printf("A %d\n", spkv_append_frame(h, 0, NULL, NULL, NULL)); break;
      case 'e':
        if (scanf("%d %d", &a1, &a2) != 2) return 1;
        printf("e %d\n", spkv_evict_frames(h, 0, c->scale_frames, c->sliding_window, a1, a2));
        break;
      case 'd':
        if (scanf("%d", &a1) != 1) return 1;
        printf("d %d\n", spkv_set_defer_eviction(h, a1));
        break;
      case 'x':
        printf("x %d\n", spkv_execute_deferred_eviction(h, 0, c->scale_frames,
                                                          c->sliding_window));
        break;
      case 'r': printf("r %d\n", spkv_rollback_last_frame(h, 0)); break;
      case 'R': printf("R %d\n", spkv_reset(h)); break;
      case 's': {
        spkv_stats st;
        rc = spkv_get_cache_stats(h, 0, &st);
        printf("s %d %lld %d %d %d %lld\n", rc, (long long)st.frame_count, (int)st.scale_pages,
               (int)st.live_pages, (int)st.free_pages, (long long)st.special_tokens);
        break;
      }
      case 'p':
        rc = spkv_plan(h, NULL);
        printf("p %d", rc);
        if (rc == SPKV_OK) {
          if (spkv_get_plan(h, table, CAP, &n_pages, &n_patch, &lpl) != SPKV_OK) return 1;
          print_list("table", table, n_pages);
          printf(" lpl %d", (int)lpl);
          if (spkv_get_plan_specials(h, runs, CAP, &n_runs) != SPKV_OK) return 1;
          print_list("pspec", runs, 3 * n_runs);
          if (spkv_get_block_specials(h, 0, runs, CAP, &n_runs) != SPKV_OK) return 1;
          print_list("bspec", runs, 3 * n_runs);
          if (spkv_get_block_state(h, 0, scale, live, free_list, CAP, &n_scale, &n_live,
                                   &n_free, &nsf) != SPKV_OK)
            return 1;
          print_list("free", free_list, n_free);
        }
        printf("\n");
        break;
      case 'c':
        printf("c %d %d %d %d %d\n", spkv_run(h, 0, NULL, NULL, nq, 0.125f, NULL),
               spkv_run_own(h, 0, NULL, NULL, nq, 0.125f, NULL, NULL, NULL),
               spkv_run_noalloc(h, 0, NULL, NULL, nq, 0.125f, NULL),
               spkv_set_num_splits(h, 3), spkv_set_num_splits(h, -1));
        break;
      default: return 1;
    }
  }
  printf("destroy %d\n", spkv_destroy(h));
  return 0;
}

int main(int argc, char** argv) {
  spkv_config c;
  spkv_handle* h = NULL;
  spkv_handle* h2 = NULL;
  static int32_t table[CAP], scale[CAP], live[CAP], free_list[CAP];
  int32_t n_pages, n_patch, lpl, n_scale, n_live, n_free;
  int64_t nsf;
  spkv_stats st;
  spkv_request req[2];
  int frames, f, rc;
  if (argc == 12 && argv[1][0] == 's') {
    c.num_blocks = atoi(argv[2]);
    c.num_heads = atoi(argv[3]);
    c.head_dim = atoi(argv[4]);
    c.page_size = atoi(argv[5]);
    c.patch_tokens = atoi(argv[6]);
    c.num_special_tokens = atoi(argv[7]);
    c.scale_frames = atoi(argv[8]);
    c.sliding_window = atoi(argv[9]);
    c.headroom = atoi(argv[10]);
    c.max_total_frames = atoi(argv[11]);
    return script(&c);
  }
  if (argc != 12) {
    fprintf(stderr, "usage: %s NB H D PS P NS S W R MTF FRAMES\n", argv[0]);
    return 2;
  }
  c.num_blocks = atoi(argv[1]);
  c.num_heads = atoi(argv[2]);
  c.head_dim = atoi(argv[3]);
  c.page_size = atoi(argv[4]);
  c.patch_tokens = atoi(argv[5]);
  c.num_special_tokens = atoi(argv[6]);
  c.scale_frames = atoi(argv[7]);
  c.sliding_window = atoi(argv[8]);
  c.headroom = atoi(argv[9]);
  c.max_total_frames = atoi(argv[10]);
  frames = atoi(argv[11]);

  {
    int64_t mnp = 0, pool = 0, wmin = 0, w1 = 0, w8 = 0;
    rc = spkv_query_sizes(&c, &mnp, &pool, &wmin);
    printf("query_sizes %d %lld %lld\n", rc, (long long)mnp, (long long)pool);
    rc = spkv_query_workspace(&c, c.num_special_tokens + c.patch_tokens, 1, &w1) ||
         spkv_query_workspace(&c, c.num_special_tokens + c.patch_tokens, 8, &w8);
    printf("query_workspace %d %d %d\n", rc, (int)(w1 > wmin), (int)(w8 - wmin > 7 * (w1 - wmin)));
    printf("query_workspace_bad %d\n", spkv_query_workspace(&c, 1, 33, &w1));
  }
  rc = spkv_create(&c, NULL, NULL, 0, &h);
  printf("create %d\n", rc);
  if (rc != SPKV_OK) return 1;
  printf("run_before_plan %d\n", spkv_run(h, 0, NULL, NULL, 1, 0.125f, NULL));
  printf("plan_empty %d\n", spkv_plan(h, NULL));
  for (f = 0; f < frames; ++f) {
    if (spkv_append_frame(h, 0, NULL, NULL, NULL) != SPKV_OK ||
        spkv_evict_frames(h, 0, c.scale_frames, c.sliding_window, 1, 0) != SPKV_OK ||
        spkv_plan(h, NULL) != SPKV_OK ||
        spkv_get_plan(h, table, CAP, &n_pages, &n_patch, &lpl) != SPKV_OK ||
        spkv_get_block_state(h, 0, scale, live, free_list, CAP, &n_scale, &n_live,
                             &n_free, &nsf) != SPKV_OK ||
        spkv_get_cache_stats(h, 0, &st) != SPKV_OK) {
      printf("frame %d failed\n", f);
      return 1;
    }
    printf("frame %d", f);
    print_list("table", table, n_pages);
    printf(" lpl %d", (int)lpl);
    print_list("free", free_list, n_free);
    printf(" stats %lld %d %d %d %lld\n", (long long)st.frame_count, (int)st.scale_pages,
           (int)st.live_pages, (int)st.free_pages, (long long)st.special_tokens);
  }
  /* checks pass on a host-only handle, then UNSUPPORTED */
  printf("run %d\n", spkv_run(h, 0, NULL, NULL, c.num_special_tokens + c.patch_tokens,
                              0.125f, NULL));
  printf("bad_block %d\n", spkv_run(h, c.num_blocks, NULL, NULL, 1, 0.125f, NULL));
  rc = spkv_create(&c, NULL, NULL, 0, &h2);
  if (rc != SPKV_OK || spkv_append_frame(h2, 0, NULL, NULL, NULL) != SPKV_OK ||
      spkv_plan(h2, NULL) != SPKV_OK)
    return 1;
  req[0].handle = h;
  req[0].block = 0;
  req[0].nq = c.num_special_tokens + c.patch_tokens;
  req[0].q = NULL;
  req[0].out = NULL;
  req[0].own_k = NULL;
  req[0].own_v = NULL;
  req[0].sm_scale = 0.125f;
  req[1] = req[0];
  req[1].handle = h2;
  printf("run_batch %d\n", spkv_run_batch(req, 2, NULL));
  req[1].handle = h;
  printf("run_batch_same_handle %d\n", spkv_run_batch(req, 2, NULL));
  printf("run_batch_empty %d\n", spkv_run_batch(req, 0, NULL));
  printf("rollback_after_evictions %d\n", spkv_rollback_last_frame(h, 0));
  printf("reset %d\n", spkv_reset(h));
  printf("run_after_reset %d\n", spkv_run(h, 0, NULL, NULL, 1, 0.125f, NULL));
  printf("destroy %d %d\n", spkv_destroy(h), spkv_destroy(h2));
  printf("error_string %s\n", spkv_error_string(SPKV_ERR_STALE_PLAN));
  return 0;
}
