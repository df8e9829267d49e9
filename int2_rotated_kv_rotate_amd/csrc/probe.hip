// Read-bandwidth probe over INT2 page records: the decode kernel's memory access pattern with
// none of its arithmetic.  Used to measure the HBM read rate that this access pattern reaches
// on the device (records of 1536 bytes at the pages a block table names, two records per step
// per wavefront, one run of records per wavefront), which is the practical ceiling of the
// decode kernel's INT2 stream.
#include "oscar_internal.h"

namespace oscar {
namespace {

constexpr int kProbeWaves = 2;

// Wavefront w reads records [w*C, min((w+1)*C, n)) of record_ids, two per step (lanes 0..63
// the first 1024 bytes of each record, lanes 0..31 the last 512), and writes the XOR of
// everything it read to out[w*64 + lane].
__global__ __launch_bounds__(64 * kProbeWaves) void read_records_kernel(
    const uint8_t* __restrict__ pool, const int32_t* __restrict__ record_ids, int n, int C,
    int workers, uint32_t* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int worker = blockIdx.x * kProbeWaves + (threadIdx.x >> 6);
  if (worker >= workers) return;
  const long long r0 = (long long)worker * C;
  const int r1 = (int)min((long long)n, r0 + C);
  uint4 acc = make_uint4(0u, 0u, 0u, 0u);
  for (int i = (int)min(r0, (long long)n); i < r1; i += 2) {
    const int ib = min(i + 1, r1 - 1);
    const uint4* ra = reinterpret_cast<const uint4*>(pool + (size_t)record_ids[i] * kRecord);
    const uint4* rb = reinterpret_cast<const uint4*>(pool + (size_t)record_ids[ib] * kRecord);
    const uint4 a0 = ra[lane], b0 = rb[lane];
    const uint4 a1 = lane < 32 ? ra[64 + lane] : make_uint4(0u, 0u, 0u, 0u);
    const uint4 b1 = lane < 32 ? rb[64 + lane] : make_uint4(0u, 0u, 0u, 0u);
    acc.x ^= a0.x ^ b0.x ^ a1.x ^ b1.x;
    acc.y ^= a0.y ^ b0.y ^ a1.y ^ b1.y;
    acc.z ^= a0.z ^ b0.z ^ a1.z ^ b1.z;
    acc.w ^= a0.w ^ b0.w ^ a1.w ^ b1.w;
  }
  out[(size_t)worker * 64 + lane] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

}  // namespace

hipError_t launch_read_records(const uint8_t* pool, const int32_t* record_ids, int n, int workers,
                               uint32_t* out, hipStream_t stream) {
  const int C = (int)((((long long)n + workers - 1) / workers + 1) & ~1LL);
  const dim3 grid((workers + kProbeWaves - 1) / kProbeWaves);
  hipLaunchKernelGGL(read_records_kernel, grid, dim3(64 * kProbeWaves), 0, stream, pool,
                     record_ids, n, C, workers, out);
  return hipGetLastError();
}

}  // namespace oscar
