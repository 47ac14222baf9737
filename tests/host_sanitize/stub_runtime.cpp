// A host-only stand-in for the HIP runtime calls the library's host code makes,
// for building api.cpp and slot_cache.cpp with g++ under AddressSanitizer and
// UndefinedBehaviorSanitizer on a machine without a GPU.  "Device" memory is
// host memory, copies are memcpy at the time of the call, streams and events
// are heap objects (so a double destroy, a use after destroy or a leak is a
// sanitizer error).  Failure injection: stub_fail_at(n) makes the n-th counted
// call from then on (every call below except hipGetErrorString,
// hipGetLastError and the destroy/free calls counts, and so does every stubbed
// kernel launch) return hipErrorLaunchFailure, once.
#include <hip/hip_runtime_api.h>

#include <cstdlib>
#include <cstring>

namespace {
long g_calls = 0;
long g_fail_at = -1;
constexpr int kLive = 0x5eed;
struct Handle {
  int live = kLive;
};
long g_handles = 0;  // events and streams not yet destroyed

template <class T>
T new_handle() {
  ++g_handles;
  return reinterpret_cast<T>(new Handle());
}
// Streams may be the null stream; events may not be null.
bool alive(const void* h, bool null_ok) {
  if (!h) return null_ok;
  return static_cast<const Handle*>(h)->live == kLive;
}
template <class T>
void destroy_handle(T h) {
  if (!h) return;
  --g_handles;
  delete reinterpret_cast<Handle*>(h);
}
}  // namespace

extern "C" void stub_fail_at(long n) {
  g_fail_at = n < 0 ? -1 : g_calls + n;
}
extern "C" long stub_calls(void) { return g_calls; }
extern "C" long stub_live_handles(void) { return g_handles; }

// Counts one call; true when it is the one chosen to fail.
extern "C" int stub_failing(void) {
  const long c = g_calls++;
  if (c == g_fail_at) {
    g_fail_at = -1;
    return 1;
  }
  return 0;
}
#define STUB_FAIL_POINT() \
  if (stub_failing()) return hipErrorLaunchFailure

extern "C" {
const char* hipGetErrorString(hipError_t e) { return e == hipSuccess ? "no error" : "stub: injected failure"; }
hipError_t hipGetLastError(void) { return hipSuccess; }
hipError_t hipGetDevice(int* d) {
  STUB_FAIL_POINT();
  *d = 0;
  return hipSuccess;
}
hipError_t hipDeviceGetAttribute(int* v, hipDeviceAttribute_t, int) {
  STUB_FAIL_POINT();
  *v = 256;
  return hipSuccess;
}
hipError_t hipMalloc(void** p, size_t n) {
  STUB_FAIL_POINT();
  *p = std::calloc(n ? n : 1, 1);
  return *p ? hipSuccess : hipErrorOutOfMemory;
}
hipError_t hipHostMalloc(void** p, size_t n, unsigned int) {
  STUB_FAIL_POINT();
  *p = std::calloc(n ? n : 1, 1);
  return *p ? hipSuccess : hipErrorOutOfMemory;
}
hipError_t hipFree(void* p) {
  std::free(p);
  return hipSuccess;
}
hipError_t hipHostFree(void* p) {
  std::free(p);
  return hipSuccess;
}
hipError_t hipHostGetDevicePointer(void** d, void* h, unsigned int) {
  STUB_FAIL_POINT();
  *d = h;
  return hipSuccess;
}
hipError_t hipMemcpy(void* dst, const void* src, size_t n, hipMemcpyKind) {
  STUB_FAIL_POINT();
  std::memmove(dst, src, n);
  return hipSuccess;
}
hipError_t hipMemcpyAsync(void* dst, const void* src, size_t n, hipMemcpyKind, hipStream_t s) {
  if (!alive(s, true)) return hipErrorInvalidHandle;
  STUB_FAIL_POINT();
  std::memmove(dst, src, n);
  return hipSuccess;
}
hipError_t hipEventCreateWithFlags(hipEvent_t* e, unsigned) {
  STUB_FAIL_POINT();
  *e = new_handle<hipEvent_t>();
  return hipSuccess;
}
hipError_t hipEventDestroy(hipEvent_t e) {
  if (!alive(e, false)) return hipErrorInvalidHandle;
  destroy_handle(e);
  return hipSuccess;
}
hipError_t hipEventRecord(hipEvent_t e, hipStream_t s) {
  if (!alive(e, false) || !alive(s, true)) return hipErrorInvalidHandle;
  STUB_FAIL_POINT();
  return hipSuccess;
}
hipError_t hipEventSynchronize(hipEvent_t e) {
  if (!alive(e, false)) return hipErrorInvalidHandle;
  STUB_FAIL_POINT();
  return hipSuccess;
}
hipError_t hipStreamWaitEvent(hipStream_t s, hipEvent_t e, unsigned int) {
  if (!alive(e, false) || !alive(s, true)) return hipErrorInvalidHandle;
  STUB_FAIL_POINT();
  return hipSuccess;
}
hipError_t hipStreamCreateWithFlags(hipStream_t* s, unsigned int) {
  STUB_FAIL_POINT();
  *s = new_handle<hipStream_t>();
  return hipSuccess;
}
hipError_t hipStreamDestroy(hipStream_t s) {
  if (!alive(s, false)) return hipErrorInvalidHandle;
  destroy_handle(s);
  return hipSuccess;
}
hipError_t hipStreamSynchronize(hipStream_t s) {
  if (!alive(s, true)) return hipErrorInvalidHandle;
  STUB_FAIL_POINT();
  return hipSuccess;
}
hipError_t hipDeviceSynchronize(void) {
  STUB_FAIL_POINT();
  return hipSuccess;
}
}  // extern "C"
