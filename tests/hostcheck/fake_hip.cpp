// Host-side stand-in for the HIP runtime functions libdpnorm imports, for a
// CPU-only build of the library's host layer under AddressSanitizer and
// UndefinedBehaviorSanitizer (test infrastructure; never part of the product).
//
// Nothing here touches a device. Kernel registration is accepted and
// ignored; a launch only checks its configuration (grid dimensions of at
// least 1 and within the hardware limits, at most 1024 threads per block) and
// counts itself; events, copies and device queries succeed without doing
// anything, and hipGetSymbolAddress returns a fixed fake address. Every
// device pointer the host layer computes is therefore only ever compared and
// offset, never dereferenced, so the sanitizers see exactly the host code.
#include <hip/hip_runtime_api.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>

extern "C" {

// referenced in place of the per-file device code objects of a host-only build
__attribute__((visibility("default"))) unsigned char dpnorm_fake_fatbin[64];

static thread_local dim3 g_grid, g_block;
static thread_local size_t g_shmem = 0;
static thread_local hipStream_t g_stream = nullptr;
static hipError_t g_last = hipSuccess;

// launch statistics, read by the fuzz driver
long long dpnorm_fake_launches = 0;
long long dpnorm_fake_bad_launches = 0;
unsigned long long dpnorm_fake_max_grid = 0;

void** __hipRegisterFatBinary(const void*) {
  static void* handle[1] = {nullptr};
  return handle;
}
void __hipRegisterFunction(void**, const void*, char*, const char*, unsigned int, void*, void*, void*, void*, int*) {}
void __hipRegisterVar(void**, void*, char*, char*, int, size_t, int, int) {}
void __hipUnregisterFatBinary(void**) {}

hipError_t __hipPushCallConfiguration(dim3 grid, dim3 block, size_t shmem, hipStream_t stream) {
  g_grid = grid;
  g_block = block;
  g_shmem = shmem;
  g_stream = stream;
  return hipSuccess;
}

hipError_t __hipPopCallConfiguration(dim3* grid, dim3* block, size_t* shmem, hipStream_t* stream) {
  *grid = g_grid;
  *block = g_block;
  *shmem = g_shmem;
  *stream = g_stream;
  return hipSuccess;
}

hipError_t hipLaunchKernel(const void*, dim3 grid, dim3 block, void**, size_t shmem, hipStream_t) {
  ++dpnorm_fake_launches;
  const unsigned long long threads = (unsigned long long)block.x * block.y * block.z;
  const bool ok = grid.x >= 1 && grid.y >= 1 && grid.z >= 1 && grid.x <= 0x7fffffffu && grid.y <= 65535u &&
                  grid.z <= 65535u && threads >= 1 && threads <= 1024 && shmem <= 160 * 1024;
  if (!ok) {
    ++dpnorm_fake_bad_launches;
    std::fprintf(stderr, "fake hipLaunchKernel: bad configuration grid (%u, %u, %u) block (%u, %u, %u) shmem %zu\n",
                 grid.x, grid.y, grid.z, block.x, block.y, block.z, shmem);
    g_last = hipErrorInvalidConfiguration;
    return g_last;
  }
  const unsigned long long g = (unsigned long long)grid.x * grid.y * grid.z;
  if (g > dpnorm_fake_max_grid) dpnorm_fake_max_grid = g;
  return hipSuccess;
}

hipError_t hipGetLastError(void) {
  const hipError_t e = g_last;
  g_last = hipSuccess;
  return e;
}

hipError_t hipEventCreate(hipEvent_t* event) {
  *event = (hipEvent_t)std::malloc(16);
  return *event ? hipSuccess : hipErrorOutOfMemory;
}
hipError_t hipEventDestroy(hipEvent_t event) {
  std::free((void*)event);
  return hipSuccess;
}
hipError_t hipEventRecord(hipEvent_t, hipStream_t) { return hipSuccess; }
hipError_t hipEventSynchronize(hipEvent_t) { return hipSuccess; }
hipError_t hipEventElapsedTime(float* ms, hipEvent_t, hipEvent_t) {
  *ms = 0.f;
  return hipSuccess;
}

hipError_t hipGetDevice(int* device) {
  *device = 0;
  return hipSuccess;
}
hipError_t hipStreamGetDevice(hipStream_t, hipDevice_t* device) {
  *device = 0;
  return hipSuccess;
}
hipError_t hipGetSymbolAddress(void** ptr, const void*) {
  *ptr = (void*)(uintptr_t)0x7e0000000000ull;
  return hipSuccess;
}
hipError_t hipMemcpyAsync(void*, const void*, size_t, hipMemcpyKind, hipStream_t) { return hipSuccess; }

}  // extern "C"
