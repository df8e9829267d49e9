// A stand-in for the few HIP runtime functions that the library's host code calls, for the
// sanitizer build of the host validation: there is no device (every query reports
// hipErrorNoDevice) and a launch only records its configuration, checks it and fails.  Linked
// into the sanitized library in place of the HIP runtime, so that build never touches a GPU.
#include <hip/hip_runtime_api.h>

#include <cstdio>

namespace {
hipError_t g_last = hipSuccess;
dim3 g_grid, g_block;
size_t g_shmem = 0;
long g_launches = 0, g_bad_launches = 0;
void* g_module = nullptr;
}  // namespace

extern "C" {

// Counters the driver reads: launches attempted, and launches whose shape was not a valid one
// (a zero grid dimension, a block of 0 or more than 1024 threads, more dynamic LDS than a CU has).
long oscar_stub_launches() { return g_launches; }
long oscar_stub_bad_launches() { return g_bad_launches; }

hipError_t hipGetDevice(int* device) {
  if (device) *device = -1;
  return g_last = hipErrorNoDevice;
}
hipError_t hipDeviceGetAttribute(int* value, hipDeviceAttribute_t, int) {
  if (value) *value = 0;
  return g_last = hipErrorNoDevice;
}
hipError_t hipOccupancyMaxActiveBlocksPerMultiprocessor(int* blocks, const void*, int, size_t) {
  if (blocks) *blocks = 0;
  return g_last = hipErrorNoDevice;
}
hipError_t hipGetSymbolAddress(void** ptr, const void*) {
  if (ptr) *ptr = nullptr;
  return g_last = hipErrorNoDevice;
}
hipError_t hipGetLastError() {
  const hipError_t e = g_last;
  g_last = hipSuccess;
  return e;
}

hipError_t __hipPushCallConfiguration(dim3 grid, dim3 block, size_t shmem, hipStream_t) {
  g_grid = grid;
  g_block = block;
  g_shmem = shmem;
  return hipSuccess;
}
hipError_t __hipPopCallConfiguration(dim3* grid, dim3* block, size_t* shmem, hipStream_t* stream) {
  *grid = g_grid;
  *block = g_block;
  *shmem = g_shmem;
  *stream = nullptr;
  return hipSuccess;
}
hipError_t hipLaunchKernel(const void*, dim3 grid, dim3 block, void**, size_t shmem, hipStream_t) {
  ++g_launches;
  const unsigned long long threads = (unsigned long long)block.x * block.y * block.z;
  if (grid.x == 0 || grid.y == 0 || grid.z == 0 || threads == 0 || threads > 1024 ||
      shmem > 160 * 1024) {
    ++g_bad_launches;
    std::fprintf(stderr, "bad launch shape: grid (%u, %u, %u) block (%u, %u, %u) lds %zu\n",
                 grid.x, grid.y, grid.z, block.x, block.y, block.z, shmem);
  }
  return g_last = hipErrorNoDevice;
}

void** __hipRegisterFatBinary(const void*) { return &g_module; }
void __hipUnregisterFatBinary(void**) {}
void __hipRegisterFunction(void**, const void*, char*, const char*, unsigned int, uint3*, uint3*,
                           dim3*, dim3*, int*) {}
void __hipRegisterVar(void**, void*, char*, char*, int, size_t, int, int) {}

}  // extern "C"
