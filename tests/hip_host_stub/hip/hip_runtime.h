// Host-only stand-in for the HIP runtime header, used to build the library's
// host code (the C ABI layer and the page-pool allocator) with g++ under the
// sanitizers.  Host-only handles (created without device buffers) never make
// a HIP call: every function here aborts, so reaching one fails the test.
#pragma once

#include <cstdio>
#include <cstdlib>

typedef int hipError_t;
enum { hipSuccess = 0, hipErrorInvalidValue = 1, hipErrorInvalidDevice = 101 };
typedef struct ihipStream_t* hipStream_t;
typedef struct ihipEvent_t* hipEvent_t;
enum hipMemcpyKind { hipMemcpyHostToDevice = 1 };
enum { hipHostMallocDefault = 0, hipEventDisableTiming = 2 };
struct hipDeviceProp_t {
  int multiProcessorCount;
};

[[noreturn]] inline void hip_host_stub_called(const char* fn) {
  std::fprintf(stderr, "HIP call %s reached on a host-only handle\n", fn);
  std::abort();
}

inline hipError_t hipGetDevice(int*) { hip_host_stub_called("hipGetDevice"); }
inline hipError_t hipSetDevice(int) { hip_host_stub_called("hipSetDevice"); }
inline hipError_t hipGetDeviceProperties(hipDeviceProp_t*, int) {
  hip_host_stub_called("hipGetDeviceProperties");
}
inline hipError_t hipHostMalloc(void**, std::size_t, unsigned) {
  hip_host_stub_called("hipHostMalloc");
}
inline hipError_t hipHostFree(void*) { hip_host_stub_called("hipHostFree"); }
inline hipError_t hipEventCreateWithFlags(hipEvent_t*, unsigned) {
  hip_host_stub_called("hipEventCreateWithFlags");
}
inline hipError_t hipEventDestroy(hipEvent_t) { hip_host_stub_called("hipEventDestroy"); }
inline hipError_t hipEventRecord(hipEvent_t, hipStream_t) {
  hip_host_stub_called("hipEventRecord");
}
inline hipError_t hipEventSynchronize(hipEvent_t) { hip_host_stub_called("hipEventSynchronize"); }
inline hipError_t hipMemcpyAsync(void*, const void*, std::size_t, hipMemcpyKind, hipStream_t) {
  hip_host_stub_called("hipMemcpyAsync");
}
