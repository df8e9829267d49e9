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
// everything it read to out[w*64 + lane].  A record id outside [0, num_records) reads the
// pool's last record instead (as the decode kernel does with page ids outside the pool); the
// second record of a step past the end of the run contributes zero.
__global__ __launch_bounds__(64 * kProbeWaves) void read_records_kernel(
    const uint8_t* __restrict__ pool, int num_records, const int32_t* __restrict__ record_ids,
    int n, int C, int workers, uint32_t* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int worker = blockIdx.x * kProbeWaves + (threadIdx.x >> 6);
  if (worker >= workers) return;
  const long long r0 = (long long)worker * C;
  const int r1 = (int)min((long long)n, r0 + C);
  const uint32_t last = (uint32_t)(num_records - 1);
  const uint4 zero = make_uint4(0u, 0u, 0u, 0u);
  uint4 acc = zero;
  for (int i = (int)min(r0, (long long)n); i < r1; i += 2) {
    // both records are always loaded (the second is record i again past the end of the run)
    // so that the four loads issue together; the dummy's words are then replaced by zeros
    const bool has_b = i + 1 < r1;
    const uint32_t ida = min((uint32_t)record_ids[i], last);
    const uint32_t idb = min((uint32_t)record_ids[has_b ? i + 1 : i], last);
    const uint4* ra = reinterpret_cast<const uint4*>(pool + (size_t)ida * kRecord);
    const uint4* rb = reinterpret_cast<const uint4*>(pool + (size_t)idb * kRecord);
    const uint4 a0 = ra[lane];
    uint4 b0 = rb[lane];
    const uint4 a1 = lane < 32 ? ra[64 + lane] : zero;
    uint4 b1 = lane < 32 ? rb[64 + lane] : zero;
    if (!has_b) {
      b0 = zero;
      b1 = zero;
    }
    acc.x ^= a0.x ^ b0.x ^ a1.x ^ b1.x;
    acc.y ^= a0.y ^ b0.y ^ a1.y ^ b1.y;
    acc.z ^= a0.z ^ b0.z ^ a1.z ^ b1.z;
    acc.w ^= a0.w ^ b0.w ^ a1.w ^ b1.w;
  }
  out[(size_t)worker * 64 + lane] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

typedef __bf16 v8bf_t __attribute__((ext_vector_type(8)));
typedef float v4f_t __attribute__((ext_vector_type(4)));

// One v_mfma_f32_16x16x32_bf16 per 16x16 tile: D = A . B + C, with A [16][32] and B [32][16]
// bf16 (row-major) and C, D [16][16] fp32.  Lane l holds row (of A) / column (of B) l % 16 and
// the 8 K indices 8 (l / 16) .. 8 (l / 16) + 7 of both operands, and D rows 4 (l / 16) + i of
// column l % 16; any pairing of the K indices that is the same in A and B gives the same
// product, so the exact value of every output is sum_k A[m][k] B[k][n] + C[m][n].
__global__ __launch_bounds__(64) void mfma_bf16_tiles_kernel(const uint16_t* __restrict__ a,
                                                             const uint16_t* __restrict__ b,
                                                             const float* __restrict__ c,
                                                             float* __restrict__ d) {
  const int l = threadIdx.x, mn = l & 15, k4 = l >> 4;
  const size_t t = blockIdx.x;
  v8bf_t av, bv;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    av[i] = __builtin_bit_cast(__bf16, a[t * 512 + mn * 32 + 8 * k4 + i]);
    bv[i] = __builtin_bit_cast(__bf16, b[t * 512 + (8 * k4 + i) * 16 + mn]);
  }
  v4f_t cv;
#pragma unroll
  for (int i = 0; i < 4; ++i) cv[i] = c[t * 256 + (4 * k4 + i) * 16 + mn];
  const v4f_t dv = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, cv, 0, 0, 0);
#pragma unroll
  for (int i = 0; i < 4; ++i) d[t * 256 + (4 * k4 + i) * 16 + mn] = dv[i];
}

}  // namespace

hipError_t launch_mfma_bf16_tiles(const uint16_t* a, const uint16_t* b, const float* c, float* d,
                                  int tiles, hipStream_t stream) {
  hipLaunchKernelGGL(mfma_bf16_tiles_kernel, dim3(tiles), dim3(64), 0, stream, a, b, c, d);
  return hipGetLastError();
}

hipError_t launch_read_records(const uint8_t* pool, int num_records, const int32_t* record_ids,
                               int n, int workers, uint32_t* out, hipStream_t stream) {
  const int C = (int)((((long long)n + workers - 1) / workers + 1) & ~1LL);
  const dim3 grid((workers + kProbeWaves - 1) / kProbeWaves);
  hipLaunchKernelGGL(read_records_kernel, grid, dim3(64 * kProbeWaves), 0, stream, pool,
                     num_records, record_ids, n, C, workers, out);
  return hipGetLastError();
}

}  // namespace oscar
