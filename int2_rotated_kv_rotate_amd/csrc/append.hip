// Rotate-clip-quantize-append: new K/V rows -> fixed orthogonal rotation -> per-token groups of
// 32 channels clipped and quantised to 2 bits -> paged INT2 records (+ BF16 sink/window rows).
//
// Method: OSCAR project card "FutureMLS-Lab/OSCAR", section "How it works" (fixed per-layer
// rotations and clipping thresholds, INT2 bulk, BF16 sink and recent window); OSCAR paper,
// "Abstract" (rotation + clipping computed offline and applied as fixed parameters; INT2 cache
// kept compatible with paged serving).  The bit-level rules (fp64 ascending accumulation of the
// rotation, fp32 scale formula, fp16 scale/zero, round-half-even codes) are this library's
// definition of the encoding and are reproduced bit for bit by the CPU oracle.
//
// This translation unit is built with -ffp-contract=off: the quantiser is an fp32 formula that
// must not be fused.
//
// Two kernels write the same bytes:
//   rotate_quantize_append_kernel (few rows, e.g. one decoded token per sequence) computes the
//     rotation as defined: fp64 on the vector ALUs, ascending channel order, one rounding to fp32;
//   rotate_quantize_prefill_kernel (many rows) computes it on the bf16 matrix cores, bounds the
//     error of every rotated value, and recomputes as defined every value whose scale, zero,
//     code or BF16 copy that bound cannot certify.
#include "oscar_internal.h"
#include "append_rows.h"

namespace oscar {
namespace {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------------ exact fp64 (few rows)
//
// The rows' rotation as defined (fp64, ascending, one rounding to fp32), then the quantiser:
// append_rows in append_rows.h, one workgroup per ROWS rows of one (KV head, K|V).

template <int ROWS>
__global__ __launch_bounds__(kAppendThreads) void rotate_quantize_append_kernel(
    CacheGeom g, uint8_t* __restrict__ pages, uint16_t* __restrict__ sinkwin,
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ slot_ids, int batch,
    int total_new, const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
    const int32_t* __restrict__ new_offsets, const int32_t* __restrict__ start_pos,
    const float* __restrict__ rot_k, const float* __restrict__ rot_v,
    const float* __restrict__ k_mean, float clip_k, float clip_v) {
  __shared__ AppendShared<ROWS> sm;
  append_rows<ROWS>(g, pages, sinkwin, block_table, slot_ids, batch, total_new, k_new, v_new,
                    new_offsets, start_pos, rot_k, rot_v, k_mean, clip_k, clip_v, blockIdx.x,
                    blockIdx.y, blockIdx.z, sm);
}

// ------------------------------------------------------------ matrix cores (many rows)
//
// A workgroup of four waves serves one (KV head, K|V) and loops over blocks of 32 rows.  Wave g
// owns group g (output channels 32g .. 32g+31) of every row of the block, so a group's
// extremes, scale, zero and codes, and the values it must recompute, stay inside one wave.  The
// wave's A operands are the rows of R^T for its channels, split exactly into three bf16 pieces
// (R = p0 + p1 + p2: 24 significand bits in three 8-bit pieces) and held in registers for the
// whole loop; the B operand is the bf16 input rows (exact), loaded from memory a block ahead.
// Twelve v_mfma_f32_16x16x32_bf16 accumulate one 16 x 16 tile into one fp32 accumulator: the p2
// pieces of the four 32-channel input slices first, then p1, then p0.  The same instruction with
// the input rows as both operands gives the diagonal of their Gram matrix, i.e. the rows'
// squared norms.
//
// Error bound.  The products are exact.  Measured on gfx950, one such instruction runs four
// passes over its 8-product blocks; a pass adds its products, aligned to the largest of them
// (bits below 2^-24 of it dropped), to the accumulator with one fp32 round-to-nearest.  Every
// product is in one block, so the dropped bits total at most 7u sum|terms| (u = 2^-24; the
// terms are the products of all three pieces, sum|terms| <= (1 + 2^-7) sum_i |x_i R_ij|).  Of
// the accumulator's 48 roundings, the 16 of the p0 passes are each at most u/2 of a partial sum
// <= sum|terms| (8u), the 32 before them act on partial sums below 2^-7 sum|terms| (0.13u), and
// the defined value's own rounding to fp32 adds u/2.  So |y_mc - y| <= 16 u sum_i |x_i R_ij| <=
// 16 u ||x|| ||R_.j||.  The coarser per-instruction bound that tests/test_gpu_mfma_model.py
// holds the device to (11u sum|products| + 4u |C| + 2^-124, C the accumulator input) gives at
// most 28u sum_i |x_i R_ij| + 12 * 2^-124 over the chain (the p0 instructions' inputs sum to at
// most 3 sum|terms|).  The kernel takes E = 64 u ||x|| ||R_.j|| plus 2^-100 for flushed
// subnormals, computed 5% high so that y -+ E rounded to nearest still encloses [y - E, y + E].
// ||x|| is bounded from the Gram diagonal: its terms are positive, so by the same model it is
// within 15u of the sum of squares, less at most 2^-122 of flushed subnormal partial sums; the
// bound takes it 1e-4 high plus 2^-121.
//
// Certification (each output is a monotone function of the values it reads):
//   * s16, z16 of a group: equal at the ends of the extremes' intervals [m - E, m + E], else
//     every channel that can hold the group's extreme (within 2E of it) is recomputed, after
//     which the extremes are the defined ones;
//   * a code: with t = (y - z) * (1/s) (fp32), the defined t lies within
//     mt = (E + (|y| + |z| + E) 2^-23) / s * 1.01 + 2^-19 of it (E, the rounding of y - z, the
//     rounding of the defined division, of 1/s and of the product, for |t| < 4); the kernel
//     takes |y| as the group's largest; the code is clamp(rint(t), 0, 3) when no half-integer
//     lies within mt of t (which includes the boundaries 1/2, 3/2, 5/2), else recomputed;
//   * a BF16 copy (sink/window row): certified when bf16(y - E) == bf16(y + E), else recomputed.
//
// Recomputation: a wave lists the values it cannot certify in LDS and recomputes them itself,
// 4 to 16 lanes per value, with R from the workgroup's copy of R^T in LDS (the midpoint argument
// at recompute_wave keeps the result the defined one).
//
// A V record holds every group's codes in each 16-bit half, so the four waves of a V workgroup
// hand their code pairs to each other through LDS once per block (one barrier); K words,
// scale/zero words and BF16 copies are written by the wave that owns the group.  With 79 KB of
// LDS (R^T in fp32 for the recomputation) two workgroups fit on a CU.
constexpr int kMWaves = kGroups;          // one wave per 32-channel group
constexpr int kMThreads = 64 * kMWaves;
constexpr int kMBlock = 32;               // rows per block: two 16-row tiles of MFMA columns
constexpr int kRtStride = kHeadDim + 4;   // floats per LDS row of R^T: the 16-byte reads of
                                          // different rows start on different banks
constexpr int kMListCap = 256;            // values a wave recomputes per round
constexpr float kErrScale = 64.0f * 0x1p-24f * 1.05f;
constexpr float kErrAbs = 0x1p-100f * 1.05f;

// The next fp32 value above / below a finite x.
__device__ __forceinline__ float up(float x) {
  if (x == 0.0f) return __uint_as_float(1u);
  const uint32_t b = __float_as_uint(x);
  return __uint_as_float(x > 0.0f ? b + 1u : b - 1u);
}
__device__ __forceinline__ float down(float x) { return -up(-x); }

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// The ||x|| bound from the Gram diagonal d2 (see above); +inf when d2 overflowed.
__device__ __forceinline__ float norm_bound(float d2) {
  return __builtin_sqrtf(d2 * 1.0001f + 0x1p-121f) * 1.0001f;
}

// Orders this wave's LDS accesses: the stores before it are complete and visible to its loads
// after it (every lane of the wave; no other wave reads these arrays).
__device__ __forceinline__ void wave_lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// A lane's value and that of lane ^ 16 (or lane ^ 32) from one lane-swap instruction (a vector
// ALU operation, no LDS round trip).  Called with both operands equal, v_permlane16_swap leaves
// each lane its own value and its partner's as the two results, own first in rows 0 and 2 of the
// wave and partner first in rows 1 and 3 (v_permlane32_swap: own first in lanes 0..31), so a
// symmetric combination (max, min, or, equality) needs no select.
struct LanePair { uint32_t a, b; };
__device__ __forceinline__ LanePair pair16(uint32_t v) {
  const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return {(uint32_t)r[0], (uint32_t)r[1]};
}
__device__ __forceinline__ LanePair pair32(uint32_t v) {
  const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return {(uint32_t)r[0], (uint32_t)r[1]};
}
// The partner's value alone.
__device__ __forceinline__ uint32_t partner16(uint32_t v, int lane) {
  const LanePair p = pair16(v);
  return (lane & 16) ? p.a : p.b;
}
__device__ __forceinline__ uint32_t partner32(uint32_t v, int lane) {
  const LanePair p = pair32(v);
  return (lane & 32) ? p.a : p.b;
}
__device__ __forceinline__ float max16(float x) {
  const LanePair p = pair16(__float_as_uint(x));
  return fmaxf(__uint_as_float(p.a), __uint_as_float(p.b));
}
__device__ __forceinline__ float min16(float x) {
  const LanePair p = pair16(__float_as_uint(x));
  return fminf(__uint_as_float(p.a), __uint_as_float(p.b));
}
__device__ __forceinline__ float max32(float x) {
  const LanePair p = pair32(__float_as_uint(x));
  return fmaxf(__uint_as_float(p.a), __uint_as_float(p.b));
}
__device__ __forceinline__ float min32(float x) {
  const LanePair p = pair32(__float_as_uint(x));
  return fminf(__uint_as_float(p.a), __uint_as_float(p.b));
}
__device__ __forceinline__ uint32_t or16(uint32_t v) { const LanePair p = pair16(v); return p.a | p.b; }
__device__ __forceinline__ uint32_t or32(uint32_t v) { const LanePair p = pair32(v); return p.a | p.b; }

struct alignas(16) MatrixShared {
  float rt[kHeadDim][kRtStride];          // R^T (fp32): rt[c][i] = R[i][c]
  double cd[kHeadDim];                    // C = mu . R (fp64, i ascending), 0 without a key mean
  float cf[kHeadDim];                     // fp32(C)
  float nrm[kMWaves][kMBlock];            // per wave: the ||x|| bound of each row of the block
  uint16_t list[kMWaves][kMListCap];      // per wave: values to recompute, 32 row + channel
  float res[kMWaves][kMListCap];          // their defined values
  uint32_t vn[2][kMWaves][kMBlock][4];    // V code pairs [buffer][group g][row]: byte c % 4 of
                                          // word c / 4 = code(32g + c) | code(32g + 16 + c) << 2
};

// Recompute n listed values of one wave as defined, L lanes per value: lane q sums the products
// of inputs (128/L) q .. (128/L)(q+1) - 1 in fp64 (exact products), and the L partial sums are
// combined.  That sum differs from the defined ascending one by at most
// 2 * 127 * 2^-53 sum|terms| <= 2^-45 ||x|| ||R_.c||, and after the fp64 subtraction of the
// key-mean term C_c (0 without a mean) by at most that plus two fp64 ulps.  Unless it lies that
// close to a midpoint between fp32 values or to zero (where the sign of a zero result is
// decided), both round to the same fp32 value, and the rare value that close is summed again in
// ascending order.  Entry k = 32 r + c (row r of the block at n0, channel c of group gq) gets its
// value in res[k].
template <int L>
__device__ __forceinline__ void recompute_wave(const uint16_t* list, float* res, int n,
                               const uint16_t* __restrict__ src, int hkv, int h, int n0, int gq,
                               const float (*rt)[kRtStride], const double* cd, const float* nrm,
                               float cng, int lane) {
  constexpr int kIn = kHeadDim / L;   // inputs per lane: 8, 16 or 32
  const int q = lane & (L - 1);
  for (int k0 = 0; k0 < n; k0 += 64 / L) {
    const int k = k0 + lane / L;
    const bool act = k < n;
    const int e = act ? list[k] : 0;
    const int r = e >> 5, c = kGroup * gq + (e & 31);
    const uint16_t* xrow = src + ((size_t)(n0 + r) * hkv + h) * kHeadDim;
    double part = 0.0, part2 = 0.0;
    if (act) {
      uint4 xv[kIn / 8];   // all of the lane's inputs in flight at once
#pragma unroll
      for (int j = 0; j < kIn / 8; ++j) xv[j] = *reinterpret_cast<const uint4*>(xrow + kIn * q + 8 * j);
#pragma unroll
      for (int j = 0; j < kIn / 8; ++j) {   // inputs kIn q + 8j .. + 7
        __builtin_amdgcn_sched_barrier(0);   // eight products at a time: few registers live
        const uint32_t xw[4] = {xv[j].x, xv[j].y, xv[j].z, xv[j].w};
        const float4* rp = reinterpret_cast<const float4*>(&rt[c][kIn * q + 8 * j]);
        const float4 r0 = rp[0], r1 = rp[1];
        const float rr[8] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
#pragma unroll
        for (int u = 0; u < 8; u += 2) {   // two chains: even and odd inputs
          part = __fma_rn((double)bf16_lo(xw[u / 2]), (double)rr[u], part);
          part2 = __fma_rn((double)bf16_hi(xw[u / 2]), (double)rr[u + 1], part2);
        }
      }
    }
    part += part2;
    part += lane_xor_f64<1>(part);
    part += lane_xor_f64<2>(part);
    if constexpr (L >= 8) {   // the other quad of the lane's eight: row_half_mirror (DPP)
      const uint64_t u = __builtin_bit_cast(uint64_t, part);
      const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, 0x141, 0xF, 0xF, true);
      const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), 0x141, 0xF, 0xF, true);
      part += __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
    }
    if constexpr (L >= 16) part += lane_xor_f64<8>(part);
    if (act && q == 0) {
      const double v = part - cd[c];
      float f = (float)v;
      const double tol = (double)nrm[r] * (double)cng * 0x1p-44 + fabs(v) * 0x1p-50;
      const double m_lo = ((double)f + (double)down(f)) * 0.5;
      const double m_hi = ((double)f + (double)up(f)) * 0.5;
      if (fabs(v - m_lo) <= tol || fabs(v - m_hi) <= tol || fabs(v) <= tol) {
        double acc = 0.0;
        for (int i = 0; i < kHeadDim; ++i)
          acc = __fma_rn((double)bf16_to_f32(xrow[i]), (double)rt[c][i], acc);
        f = (float)(acc - cd[c]);
      }
      res[k] = f;
    }
  }
}

// Inclusive prefix sum over the wave's lanes (row shifts within 16-lane rows, then the row
// broadcasts of lanes 15 and 31).
__device__ __forceinline__ int wave_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, true);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, true);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, true);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, true);   // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);  // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return x;
}

// The 16 values' codes of a lane: 2 bits each (INT2 records) or 4 (INT4 records), value v at
// bits BITS * v.
template <int BITS>
struct CodeWord { using T = uint32_t; };
template <>
struct CodeWord<4> { using T = uint64_t; };

// INT4 records (2560 bytes, the layout of the INT4 append): K codes [0, 1024), V codes
// [1024, 2048), K (scale, zero) [2048, 2304), V [2304, 2560).
constexpr int kRecord4 = 2560, kK4Codes = 0, kV4Codes = 1024, kK4Meta = 2048, kV4Meta = 2304;

// Replace this wave's flagged values by the defined ones.  Bit v = 8 tb + 4 cb + i of fl: the
// lane's value y[v], row 16 tb + m of the block, channel 16 cb + 4 kq + i of the group.  The
// wave's flagged values are numbered lane first, then value index, and recomputed in rounds of
// up to kMListCap.  RECODE: also replace their codes (bits BITS v of cw) by the defined ones,
// with the rows' scale sc and zero zz.
template <int BITS, bool RECODE>
__device__ __forceinline__ void recompute_flagged(uint32_t fl, float (&y)[16],
                                                  typename CodeWord<BITS>::T& cw,
                                                  const float sc[2], const float zz[2],
                                                  uint16_t* list, float* res,
                                                  const uint16_t* __restrict__ src, int hkv, int h,
                                                  int n0, int gq, const float (*rt)[kRtStride],
                                                  const double* cd, const float* nrm, float cng,
                                                  int lane) {
  const int m = lane & 15, kq = lane >> 4;
  const int cnt = __builtin_popcount(fl);
  const int incl = wave_scan(cnt);
  const int excl = incl - cnt;
  const int total = __builtin_amdgcn_readlane(incl, 63);
  uint32_t wor = fl;   // the value indices flagged in any lane
  wor |= lane_xor<1>(wor);
  wor |= lane_xor<2>(wor);
  wor |= lane_xor<4>(wor);
  wor |= lane_xor<8>(wor);
  wor = or16(wor);
  wor = or32(wor);
  wor = __builtin_amdgcn_readfirstlane(wor);
  for (int r0 = 0; r0 < total; r0 += kMListCap) {
    {
      uint32_t f = fl;
      int p = excl - r0;
      while (f != 0u) {
        const int v = __builtin_ctz(f);
        f &= f - 1u;
        if (p >= 0 && p < kMListCap)
          list[p] = (uint16_t)(kGroup * (16 * (v >> 3) + m) + 16 * ((v >> 2) & 1) + 4 * kq + (v & 3));
        ++p;
      }
    }
    wave_lds_sync();
    // as many lanes per value as fill the wave in one step (at least 4)
    const int nr = min(kMListCap, total - r0);
    if (nr <= 4)
      recompute_wave<16>(list, res, nr, src, hkv, h, n0, gq, rt, cd, nrm, cng, lane);
    else if (nr <= 8)
      recompute_wave<8>(list, res, nr, src, hkv, h, n0, gq, rt, cd, nrm, cng, lane);
    else
      recompute_wave<4>(list, res, nr, src, hkv, h, n0, gq, rt, cd, nrm, cng, lane);
    wave_lds_sync();
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      if ((wor >> v) & 1u) {
        const int p = excl + __builtin_popcount(fl & ((1u << v) - 1u)) - r0;
        if (((fl >> v) & 1u) && p >= 0 && p < kMListCap) {
          y[v] = res[p];
          if (RECODE) {
            using T = typename CodeWord<BITS>::T;
            constexpr int kSteps = (1 << BITS) - 1;
            const int code = code_of_t<kSteps>(y[v], v >> 3 ? sc[1] : sc[0], v >> 3 ? zz[1] : zz[0]);
            cw = (cw & ~((T)kSteps << (BITS * v))) | ((T)code << (BITS * v));
          }
        }
      }
    }
    wave_lds_sync();
  }
}

// Group extremes of the lane's rows (tb = 0, 1) over the four lanes kq of each row.
__device__ __forceinline__ void group_extremes(const float (&y)[16], float mx[2], float mn[2]) {
#pragma unroll
  for (int tb = 0; tb < 2; ++tb) {
    float a = y[8 * tb], b = y[8 * tb];
#pragma unroll
    for (int j = 1; j < 8; ++j) {
      a = fmaxf(a, y[8 * tb + j]);
      b = fminf(b, y[8 * tb + j]);
    }
    a = max32(max16(a));
    b = min32(min16(b));
    mx[tb] = a;
    mn[tb] = b;
  }
}

// Sequence of flattened new row n: the largest b < batch with off[b] <= n, searched upward
// from `seq` (a sequence of an earlier row), galloping then bisecting; bounded loops.
__device__ int advance_seq(const int32_t* __restrict__ off, int batch, int seq, int n) {
  int lo = seq, hi;
  int step = 1;
  for (int i = 0; i < 32; ++i) {
    hi = lo + step;
    if (hi >= batch) { hi = batch; break; }
    if (off[hi] > n) break;
    lo = hi;
    step <<= 1;
  }
  for (int i = 0; i < 32 && hi - lo > 1; ++i) {
    const int mid = lo + (hi - lo) / 2;
    if (off[mid] <= n) lo = mid;
    else hi = mid;
  }
  return lo;
}

// BITS = 2: INT2 records; BITS = 4: INT4 records (16 levels, the INT4 append's layout).
template <int BITS>
__global__ __launch_bounds__(kMThreads, 2) void rotate_quantize_prefill_kernel(
    CacheGeom g, uint8_t* __restrict__ pages, uint16_t* __restrict__ sinkwin,
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ slot_ids, int batch,
    int total_new, const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
    const int32_t* __restrict__ new_offsets, const int32_t* __restrict__ start_pos,
    const float* __restrict__ rot_k, const float* __restrict__ rot_v,
    const float* __restrict__ k_mean, float clip_k, float clip_v, int k_groups) {
#pragma clang fp contract(off)
  __shared__ MatrixShared sm;
  const int t = threadIdx.x, lane = t & 63;
  const int gq = __builtin_amdgcn_readfirstlane(t >> 6);   // this wave's group
  const int h = blockIdx.y;
  // workgroups [0, k_groups) of a KV head serve its K rows, the rest its V rows; x0 is this
  // workgroup's index among the G of its (head, K|V) pair
  const bool is_v = (int)blockIdx.x >= k_groups;
  const int G = is_v ? (int)gridDim.x - k_groups : k_groups;
  const int x0 = is_v ? (int)blockIdx.x - k_groups : (int)blockIdx.x;
  const float* rot = (is_v ? rot_v : rot_k) + (size_t)h * kHeadDim * kHeadDim;
  const uint16_t* src = is_v ? v_new : k_new;
  const float clip = is_v ? clip_v : clip_k;
  const bool centered = !is_v && k_mean != nullptr;
  const bool has_store = sinkwin != nullptr;
  const int m = lane & 15, kq = lane >> 4;
  constexpr int kSteps = (1 << BITS) - 1;
  constexpr int kRec = BITS == 2 ? kRecord : kRecord4;
  using CW = typename CodeWord<BITS>::T;

  // Stage R^T: all 16 float4 loads of a thread first, then the transposed LDS stores.
  {
    constexpr int kPer = kHeadDim * kHeadDim / 4 / kMThreads;  // 16
    const float4* rot4 = reinterpret_cast<const float4*>(rot);
    float4 rr[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) rr[k] = rot4[t + kMThreads * k];
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int e = 4 * (t + kMThreads * k), i = e / kHeadDim, j = e % kHeadDim;
      sm.rt[j][i] = rr[k].x;
      sm.rt[j + 1][i] = rr[k].y;
      sm.rt[j + 2][i] = rr[k].z;
      sm.rt[j + 3][i] = rr[k].w;
    }
  }
  __syncthreads();

  // The group's largest column norm (rounded up) and key-mean terms: lane l takes column
  // 32g + l % 32 (the upper half of the wave repeats the lower).
  float cng, cmax;
  {
    const int c = kGroup * gq + (lane & 31);
    float ss = 0.f;
    double cdv = 0.0;
    for (int i = 0; i < kHeadDim; ++i) ss = fmaf(sm.rt[c][i], sm.rt[c][i], ss);
    if (centered)   // C_c = sum_i mu_i R_ic, fp64, i ascending (exact products)
      for (int i = 0; i < kHeadDim; ++i)
        cdv = __fma_rn((double)k_mean[(size_t)h * kHeadDim + i], (double)sm.rt[c][i], cdv);
    if (lane < 32) {
      sm.cd[c] = cdv;
      sm.cf[c] = (float)cdv;
    }
    float cm = fabsf((float)cdv);
    ss = fmaxf(ss, lane_xor_f32<1>(ss));
    cm = fmaxf(cm, lane_xor_f32<1>(cm));
    ss = fmaxf(ss, lane_xor_f32<2>(ss));
    cm = fmaxf(cm, lane_xor_f32<2>(cm));
    ss = fmaxf(ss, lane_xor_f32<4>(ss));
    cm = fmaxf(cm, lane_xor_f32<4>(cm));
    ss = fmaxf(ss, lane_xor_f32<8>(ss));
    cm = fmaxf(cm, lane_xor_f32<8>(cm));
    ss = fmaxf(ss, lane_xor_f32<16>(ss));
    cm = fmaxf(cm, lane_xor_f32<16>(cm));
    cng = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(__builtin_sqrtf(ss) * 1.001f)));
    cmax = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(cm)));
  }
  __syncthreads();
  // A operands: lane (m, kq), channel block cb, slice s holds R[32s + 8kq + e][32g + 16cb + m],
  // e = 0..7, as 3 pieces.
  v8bf ra[2][4][3];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb)
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const float* rp = &sm.rt[kGroup * gq + 16 * cb + m][32 * s + 8 * kq];
      const float4 r0 = *reinterpret_cast<const float4*>(rp);
      const float4 r1 = *reinterpret_cast<const float4*>(rp + 4);
      const float rv[8] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
      uint16_t pc[3][8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        pc[0][e] = f32_to_bf16_rne(rv[e]);
        const float d1 = rv[e] - bf16_to_f32(pc[0][e]);
        pc[1][e] = f32_to_bf16_rne(d1);
        pc[2][e] = f32_to_bf16_rne(d1 - bf16_to_f32(pc[1][e]));
      }
#pragma unroll
      for (int p = 0; p < 3; ++p) {
        uint4 w;
        w.x = pc[p][0] | ((uint32_t)pc[p][1] << 16);
        w.y = pc[p][2] | ((uint32_t)pc[p][3] << 16);
        w.z = pc[p][4] | ((uint32_t)pc[p][5] << 16);
        w.w = pc[p][6] | ((uint32_t)pc[p][7] << 16);
        ra[cb][s][p] = __builtin_bit_cast(v8bf, w);
      }
    }

  const int ntiles = (total_new + kMBlock - 1) / kMBlock;
  // Block order: round k takes tile k * G + (x + k) mod G (G workgroups per pair, x this one),
  // one tile of each span of G; the rotation spreads tiles that cost more (the last rows of
  // every sequence, whose BF16 copies are certified too) over all workgroups.  Successive tiles
  // of a workgroup increase, as the placement look-ahead needs.
  auto tile_of = [&](int k) { return k * G + (x0 + k) % G; };   // tile_of(0) == x0

  // B operands of a block: lane (m, kq), row 16 tb + m, slice s holds inputs 32s + 8kq .. +7.
  // A row past the end (or past the last block) loads the last row instead: its values are
  // never stored and no flag is raised for it, and the loads stay unconditional, so a later
  // wait for an earlier load can count them exactly instead of waiting for all.
  uint4 xs[2][4];
  auto load_x = [&](int tile) {
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      const int n = min(tile * kMBlock + 16 * tb + m, total_new - 1);
      const uint4* rp = reinterpret_cast<const uint4*>(src + ((size_t)n * g.hkv + h) * kHeadDim + 8 * kq);
#pragma unroll
      for (int s = 0; s < 4; ++s) xs[tb][s] = rp[4 * s];
    }
  };

  // This lane looks up the placement of block row tp; the other row it holds comes from lane
  // kq ^ 1.  The lookups of the next block run a stage per phase (one dependent load each).
  const int tp = 16 * (kq & 1) + m;
  int seq = 0;
  RowInfo info_next{-1, 0, -1};
  if (x0 < ntiles && x0 * kMBlock + tp < total_new) {
    const int n = x0 * kMBlock + tp;
    seq = row_to_seq(new_offsets, batch, n);
    info_next = row_info_t<kRec>(g, block_table, slot_ids, batch, new_offsets, start_pos, has_store,
                                 n, h, is_v);
  }
  load_x(x0);
  uint16_t* list = sm.list[gq];
  float* res = sm.res[gq];
  const float* nrm_w = sm.nrm[gq];

  for (int k = 0, tile = x0; tile < ntiles; ++k, tile = tile_of(k)) {
    const int n0 = tile * kMBlock;
    const int nt = tile_of(k + 1);     // the successor block
    const int n_next = nt * kMBlock + tp;
    const bool look = nt < ntiles && n_next < total_new;
    // placement of row tp (this lane's row of block tile tp / 16), and the BF16-copy offsets of
    // both its rows (tb = 0, 1)
    const RowInfo own = info_next;
    long long sw[2];
    {
      const long long so = (long long)(((uint64_t)partner16((uint32_t)((uint64_t)own.sw >> 32), lane) << 32) |
                                       partner16((uint32_t)own.sw, lane));
      sw[0] = (kq & 1) ? so : own.sw;
      sw[1] = (kq & 1) ? own.sw : so;
    }
    bool valid[2];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) valid[tb] = n0 + 16 * tb + m < total_new;

    // placement stage 1: is the successor's row still in the same sequence?
    int off_up = 0;
    if (look && seq + 1 < batch) off_up = new_offsets[seq + 1];

    // y and the rows' norm bounds on the matrix cores
    float y[16], nrm[2];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      __builtin_amdgcn_sched_barrier(0);   // one 16-row tile's chains at a time
      v8bf xb[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) xb[s] = __builtin_bit_cast(v8bf, xs[tb][s]);
      v4f gm = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) gm = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xb[s], xb[s], gm, 0, 0, 0);
      // lane (m, kq) holds Gram rows 4kq .. 4kq+3 of column m: the diagonal entry of row m is in
      // lane (m, m / 4), element m % 4
      const int mi = m & 3;
      const float d = mi == 0 ? gm[0] : mi == 1 ? gm[1] : mi == 2 ? gm[2] : gm[3];
      nrm[tb] = norm_bound(__shfl(d, m + 16 * (m >> 2)));
      v4f a[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int pc = 2; pc >= 0; --pc)
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
          for (int cb = 0; cb < 2; ++cb)
            a[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ra[cb][s][pc], xb[s], a[cb], 0, 0, 0);
      // D row = channel 16cb + 4kq + i of the group, column = row 16tb + m of the block
#pragma unroll
      for (int cb = 0; cb < 2; ++cb)
#pragma unroll
        for (int i = 0; i < 4; ++i) y[8 * tb + 4 * cb + i] = a[cb][i];
      if (centered) {   // minus fp32(C) of the lane's channels 32g + 16cb + 4kq + i
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
          const float4 cf = *reinterpret_cast<const float4*>(&sm.cf[kGroup * gq + 16 * cb + 4 * kq]);
          y[8 * tb + 4 * cb] -= cf.x;
          y[8 * tb + 4 * cb + 1] -= cf.y;
          y[8 * tb + 4 * cb + 2] -= cf.z;
          y[8 * tb + 4 * cb + 3] -= cf.w;
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    if (kq == 0) {
      sm.nrm[gq][m] = nrm[0];
      sm.nrm[gq][16 + m] = nrm[1];
    }

    // placement stage 2: the successor row's sequence, then its per-sequence values
    int first = 0, next_first = 0, sp = 0, slot = 0;
    if (look) {
      if (seq + 1 < batch && off_up <= n_next) seq = advance_seq(new_offsets, batch, seq + 1, n_next);
      first = new_offsets[seq];
      next_first = new_offsets[seq + 1];
      sp = start_pos[seq];
      slot = slot_ids ? slot_ids[seq] : seq;
    }

    // Pass 1: certify each group's scale and zero; where they are not certain, flag every
    // channel that can hold the group's maximum or minimum.  Lane kq evaluates one end of one
    // row's interval: row tb = kq / 2, upper ends for even kq.
    float mx[2], mn[2], E[2];
    group_extremes(y, mx, mn);
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
      E[tb] = kErrScale * nrm[tb] * cng + kErrAbs +
              (centered ? (cmax + 2.0f * fmaxf(fabsf(mx[tb]), fabsf(mn[tb]))) * 0x1p-22f : 0.0f);
    uint32_t unsure;
    {
      const int vt = kq >> 1;
      const bool lo_end = (kq & 1) != 0;
      const float a = vt ? mx[1] : mx[0], b = vt ? mn[1] : mn[0], e = vt ? E[1] : E[0];
      _Float16 s16, z16;
      group_params_t<kSteps>(lo_end ? a - e : a + e, lo_end ? b + e : b - e, clip, s16, z16);
      const uint32_t key = meta_word(s16, z16);
      const LanePair ends = pair16(key);                            // kq ^ 1: the other end
      const uint32_t diff = ends.a != ends.b ? 1u : 0u;
      const uint32_t other = partner32(diff, lane);                 // kq ^ 2: the other row
      unsure = (diff << vt) | (other << (vt ^ 1));
    }
    uint32_t fl = 0;
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      if (((unsure >> tb) & 1u) && valid[tb]) {
        const float top = mx[tb] - 2.0f * E[tb], bot = mn[tb] + 2.0f * E[tb];
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (y[8 * tb + j] >= top || y[8 * tb + j] <= bot) fl |= 1u << (8 * tb + j);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    CW cw = 0;   // codes at bits BITS v
    const bool redo = __ballot(fl != 0u) != 0;
    if (redo) {
      const float none[2] = {0.f, 0.f};
      recompute_flagged<BITS, false>(fl, y, cw, none, none, list, res, src, g.hkv, h, n0, gq, sm.rt,
                               sm.cd, nrm_w, cng, lane);
    }
    __builtin_amdgcn_sched_barrier(0);

    // placement stage 3: page of the successor row
    int pos = 0, page = -1;
    if (look) {
      pos = sp + (n_next - first);
      const int lp = pos / kPage;
      if (pos >= 0 && lp < g.max_pages) page = block_table[(size_t)seq * g.max_pages + lp];
    }

    // Pass 2: the group's scale and zero (now the defined ones), every code and BF16 copy; flag
    // what the bound cannot certify (E taken for the group's largest column norm).  Lane kq
    // evaluates row kq % 2's scale and zero.  (Values recomputed in pass 1 are certified with
    // the same margins as the others: looser than they need, never wrong.)
    if (redo) group_extremes(y, mx, mn);
    uint32_t meta[2];
    float sc[2], zz[2], inv[2];
    {
      const int pt = kq & 1;
      _Float16 s16, z16;
      group_params_t<kSteps>(pt ? mx[1] : mx[0], pt ? mn[1] : mn[0], clip, s16, z16);
      const uint32_t mw = meta_word(s16, z16);
      const float s = (float)s16;
      const float iv = s != 0.0f ? 1.0f / s : 0.0f;
      const uint32_t mo = partner16(mw, lane);
      const float io = __uint_as_float(partner16(__float_as_uint(iv), lane));
      meta[0] = pt ? mo : mw;
      meta[1] = pt ? mw : mo;
      inv[0] = pt ? io : iv;
      inv[1] = pt ? iv : io;
    }
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      sc[tb] = (float)__builtin_bit_cast(_Float16, (uint16_t)meta[tb]);
      zz[tb] = (float)__builtin_bit_cast(_Float16, (uint16_t)(meta[tb] >> 16));
    }
    if (kq < 2) {   // lane kq stores row kq's scale/zero word of the group
      if ((kq ? valid[1] : valid[0]) && own.rec >= 0) {
        if constexpr (BITS == 2) {
          store_meta(pages, own, is_v, gq, kq ? meta[1] : meta[0]);
        } else {
          *reinterpret_cast<uint32_t*>(pages + own.rec + (is_v ? kV4Meta : kK4Meta) +
                                       16 * own.slot_in_page + 4 * gq) = kq ? meta[1] : meta[0];
        }
      }
    }
    uint32_t fl2 = 0;   // values to recompute
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      const float Eg = kErrScale * nrm[tb] * cng + kErrAbs +
                       (centered ? (cmax + 2.0f * fmaxf(fabsf(mx[tb]), fabsf(mn[tb]))) * 0x1p-22f : 0.0f);
      // the code margin of the group, taken at its largest |y| (>= every |y| in it).  The
      // computed t carries three fp32 roundings (the difference, 1/s and the product) beyond the
      // defined quotient's one: 4u |y - z| / s, with |y - z| <= gabs; with 4 levels the 2^-23
      // term and the 2^-19 floor cover it (|t| that large needs gabs >> |y - z|), with 16 levels
      // the relative term is 2^-22.
      const float gabs = fmaxf(fabsf(mx[tb]), fabsf(mn[tb])) + fabsf(zz[tb]);
      constexpr float kRel = BITS == 2 ? 0x1p-23f : 0x1p-22f;
      const float mt = (Eg + (gabs + Eg) * kRel) * inv[tb] * 1.01f + 0x1p-19f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int v = 8 * tb + j;
        const float yv = y[v];
        // t within mt of the defined t; the code is certain when no boundary 1/2, 3/2, 5/2
        // lies within mt of t.  The distance to the nearest half-integer is at most the
        // distance to those three, so comparing it is conservative.
        const float tq = (yv - zz[tb]) * inv[tb];
        const float dist = fabsf(__builtin_amdgcn_fractf(tq) - 0.5f);
        const bool ok = dist > mt;
        const int code = (int)fminf(fmaxf(__builtin_rintf(tq), 0.0f), (float)kSteps);
        cw |= (CW)code << (BITS * v);
        fl2 |= (ok ? 0u : 1u) << v;
      }
      // BF16 copies of sink/window rows: certain when y -+ E round to the same bf16
      if (__ballot(sw[tb] >= 0) != 0 && sw[tb] >= 0) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int v = 8 * tb + j;
          if (f32_to_bf16_rne(y[v] - Eg) != f32_to_bf16_rne(y[v] + Eg)) fl2 |= 1u << v;
        }
      }
      if (!valid[tb]) fl2 &= ~(0xFFu << (8 * tb));
    }
    __builtin_amdgcn_sched_barrier(0);
    if (__ballot(fl2 != 0u) != 0)
      recompute_flagged<BITS, true>(fl2, y, cw, sc, zz, list, res, src, g.hkv, h, n0, gq, sm.rt, sm.cd,
                              nrm_w, cng, lane);

    load_x(nt);   // the successor's rows, in flight from here to the next block's matrix cores
    // placement stage 4: the successor row's record and sink/window row
    if (look) {
      RowInfo nx{-1, 0, -1};
      if (pos >= 0 && page >= 0 && page < g.num_pages && pos / kPage < g.max_pages) {
        nx.rec = ((long long)page * g.hkv + h) * kRec;
        nx.slot_in_page = pos % kPage;
      }
      const int new_len = sp + (next_first - first);
      int row = -1;
      if (pos >= 0 && pos < g.num_sink) row = pos;
      else if (g.window > 0 && pos >= g.num_sink && pos >= new_len - g.window)
        row = g.num_sink + pos % g.window;
      if (row >= 0 && has_store && slot >= 0 && slot < g.num_slots)
        nx.sw = (((long long)slot * g.hkv + h) * (g.num_sink + g.window) + row) * 2 * kHeadDim +
                (is_v ? kHeadDim : 0);
      info_next = nx;
    } else {
      info_next = RowInfo{-1, 0, -1};
    }

    // BF16 copies of sink/window rows: lane (m, kq) holds 4 consecutive channels per block cb
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      if (valid[tb] && sw[tb] >= 0) {
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
          const int v = 8 * tb + 4 * cb;
          const uint2 o = {(uint32_t)f32_to_bf16_rne(y[v]) | ((uint32_t)f32_to_bf16_rne(y[v + 1]) << 16),
                           (uint32_t)f32_to_bf16_rne(y[v + 2]) | ((uint32_t)f32_to_bf16_rne(y[v + 3]) << 16)};
          *reinterpret_cast<uint2*>(sinkwin + sw[tb] + kGroup * gq + 16 * cb + 4 * kq) = o;
        }
      }
    }

    if constexpr (BITS == 2) {
      if (!is_v) {
        // K word d = 2g + cb of row 16 tb + m: channel 4kq + i of the word at bits 8kq + 2i, so
        // the four lanes of a row contribute a byte each; lane kq stores word cb = kq / 2 of its
        // own row (tb = kq % 2)
        uint32_t wsel = 0;
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
          for (int cb = 0; cb < 2; ++cb) {
            uint32_t w = ((cw >> (16 * tb + 8 * cb)) & 0xFFu) << (8 * kq);
            w = or32(or16(w));
            if (kq == 2 * cb + tb) wsel = w;
          }
        if (((kq & 1) ? valid[1] : valid[0]) && own.rec >= 0) {
          const int d = 2 * gq + (kq >> 1);
          *reinterpret_cast<uint32_t*>(pages + own.rec + kKCodes + 8 * (16 * (d % 4) + own.slot_in_page) +
                                       4 * (d / 4)) = wsel;
        }
      } else {
        // V: the group's code pairs of channel residues c16 = 4kq + i, to LDS, then each thread
        // assembles two 16-bit halves of one row from the four groups' pairs
        const int buf = k & 1;
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
          uint32_t wv = 0;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint32_t nib = ((cw >> (16 * tb + 2 * i)) & 3u) | (((cw >> (16 * tb + 8 + 2 * i)) & 3u) << 2);
            wv |= nib << (8 * i);
          }
          sm.vn[buf][gq][16 * tb + m][kq] = wv;
        }
        __syncthreads();
        const int tl = t >> 3, c2 = 2 * (t & 7);
        // row tl's placement is held by lane (tl % 16, tl / 16) of every wave
        const int srcl = (tl & 15) + 16 * (tl >> 4);
        const uint32_t rlo = (uint32_t)__shfl((int)(uint32_t)own.rec, srcl);
        const uint32_t rhi = (uint32_t)__shfl((int)(uint32_t)((uint64_t)own.rec >> 32), srcl);
        const int sl = __shfl(own.slot_in_page, srcl);
        const long long rec = (long long)(((uint64_t)rhi << 32) | rlo);
        if (n0 + tl < total_new && rec >= 0) {
          uint32_t hw0 = 0, hw1 = 0;
#pragma unroll
          for (int gg = 0; gg < kMWaves; ++gg) {
            const uint32_t wv = sm.vn[buf][gg][tl][c2 >> 2];
            hw0 |= ((wv >> (8 * (c2 & 3))) & 0xFu) << (4 * gg);
            hw1 |= ((wv >> (8 * ((c2 + 1) & 3))) & 0xFu) << (4 * gg);
          }
          uint8_t* base = pages + rec + kVCodes + 4 * ((sl % 4) / 2) + 2 * (sl % 2);
          *reinterpret_cast<uint16_t*>(base + 8 * (16 * (sl / 4) + c2)) = (uint16_t)hw0;
          *reinterpret_cast<uint16_t*>(base + 8 * (16 * (sl / 4) + c2 + 1)) = (uint16_t)hw1;
        }
      }
    } else if (!is_v) {
      // INT4 K: channel 4kq + i of block cb goes to chunk 16 q + slot (q = 2 (g % 2) + cb), byte
      // 8 (g / 2) + 4 (i / 2) + kq, nibble i % 2: the four lanes of a row contribute a byte of
      // each of the two dwords; lane kq stores both dwords of (tb, cb) = (kq % 2, kq / 2) of its
      // own row
      uint2 wsel = {0u, 0u};
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
          const int vb = 8 * tb + 4 * cb;
          uint32_t w0 = ((uint32_t)(cw >> (4 * vb)) & 0xFFu) << (8 * kq);
          uint32_t w1 = ((uint32_t)(cw >> (4 * vb + 8)) & 0xFFu) << (8 * kq);
          w0 = or32(or16(w0));
          w1 = or32(or16(w1));
          if (kq == 2 * cb + tb) wsel = make_uint2(w0, w1);
        }
      if (((kq & 1) ? valid[1] : valid[0]) && own.rec >= 0) {
        const int q = 2 * (gq & 1) + (kq >> 1);
        *reinterpret_cast<uint2*>(pages + own.rec + kK4Codes + 16 * (16 * q + own.slot_in_page) +
                                  8 * (gq >> 1)) = wsel;
      }
    } else {
      // INT4 V: channel 4kq + i of blocks cb = 0, 1 share a byte (cb in the nibble) of dword g in
      // chunk 16 (slot / 4) + 4kq + i, byte 2 (u % 2) + u / 2 (u = slot % 4): each slot owns whole
      // bytes, so no exchange between groups.  A lane stores its own row's bytes of its channels
      // and, from lane kq ^ 1 (which holds the other row), those of that lane's channels.
      uint32_t vb[2];   // [tb]: byte i of channel 4kq + i at bits 8i
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        uint32_t b = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t lo = (uint32_t)(cw >> (4 * (8 * tb + i))) & 0xFu;
          const uint32_t hi = (uint32_t)(cw >> (4 * (8 * tb + 4 + i))) & 0xFu;
          b |= (lo | (hi << 4)) << (8 * i);
        }
        vb[tb] = b;
      }
      const uint32_t mine = (kq & 1) ? vb[1] : vb[0];
      const uint32_t theirs = partner16((kq & 1) ? vb[0] : vb[1], lane);
      if (((kq & 1) ? valid[1] : valid[0]) && own.rec >= 0) {
        const int sl = own.slot_in_page, u = sl & 3;
        uint8_t* base = pages + own.rec + kV4Codes + 16 * (16 * (sl >> 2)) + 4 * gq + 2 * (u & 1) +
                        (u >> 1);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          base[16 * (4 * kq + i)] = (uint8_t)(mine >> (8 * i));
          base[16 * (4 * (kq ^ 1) + i)] = (uint8_t)(theirs >> (8 * i));
        }
      }
    }
  }
}

// ------------------------------------------------------------------ Hadamard rotation
//
// R = diag(s) . H / sqrt(128) with H the Sylvester-Hadamard matrix of order 128: the signed row
// goes through the fast Walsh-Hadamard transform in fp64 (stages h = 1, 2, ..., 64, the pair
// (u_i, u_{i+h}) becoming (u_i + u_{i+h}, u_i - u_{i+h})), each result is multiplied in fp64 by
// the double nearest to 1/sqrt(128) and rounded to fp32.  896 additions per row instead of
// 16,384 multiply-adds, so no matrix and no certification.
//
// Sixteen lanes per row, four rows per wavefront at a time: row slot q = lane / 16, lane
// l = lane % 16 of the slot.  Layout A, lane l holding channels 8l .. 8l + 7, keeps stages
// h = 1, 2, 4 inside the lane; an LDS transpose gives layout B, lane l holding channels
// l + 16e (e = 0..7), where h = 16, 32, 64 are inside the lane and h = 8 pairs lane l with lane
// l ^ 8 (a DPP row rotation).  The fp32 results go back to layout A through LDS, where the
// four lanes 4g .. 4g + 3 hold quantisation group g.  Each row slot takes a contiguous quarter
// of the wavefront's rows (sequence, page and slot advanced incrementally, the next page id
// read ahead), and the next kHadAhead rows of every slot are loaded while the current ones are
// computed.

constexpr double kHadScale = 0x1.6a09e667f3bcdp-4;   // the double nearest to 2^-3.5 (sqrt(2)/16)
constexpr int kHadWaves = 4;
constexpr int kHadAhead = 2;
constexpr int kHadStrideD = kHeadDim + 2;   // doubles per row slot in the transpose buffer
constexpr int kHadStrideF = kHeadDim + 4;   // floats per row slot

struct HadShared {
  double d[kHadWaves][4][kHadStrideD];      // layout A -> B (fp64)
  float f[kHadWaves][4][kHadStrideF];       // layout B -> A (fp32 results)
};

// x with its sign flipped where sign has bit 31 set (exact).
__device__ __forceinline__ double with_sign(double x, uint32_t sign) {
  uint64_t u = __builtin_bit_cast(uint64_t, x);
  u ^= (uint64_t)sign << 32;
  return __builtin_bit_cast(double, u);
}
// In-lane FWHT pair: (a, b) -> (a + b, a - b).
__device__ __forceinline__ void fwht_pair(double& a, double& b) {
  const double s = a + b, d = a - b;
  a = s;
  b = d;
}

__global__ __launch_bounds__(64 * kHadWaves) void rotate_quantize_hadamard_kernel(
    CacheGeom g, uint8_t* __restrict__ pages, uint16_t* __restrict__ sinkwin,
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ slot_ids, int batch,
    int total_new, const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
    const int32_t* __restrict__ new_offsets, const int32_t* __restrict__ start_pos,
    const int8_t* __restrict__ signs_k, const int8_t* __restrict__ signs_v, float clip_k,
    float clip_v) {
#pragma clang fp contract(off)
  __shared__ HadShared sm;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int q = lane >> 4, l = lane & 15;
  const int h = blockIdx.y;
  const bool is_v = blockIdx.z != 0;
  const uint16_t* src = is_v ? v_new : k_new;
  const int8_t* sg = is_v ? signs_v : signs_k;
  const float clip = is_v ? clip_v : clip_k;
  uint32_t neg = 0;  // bit e: channel 8l + e is negated
  if (sg != nullptr) {
    const uint2 s8 = *reinterpret_cast<const uint2*>(sg + h * kHeadDim + 8 * l);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t byte = ((e < 4 ? s8.x : s8.y) >> (8 * (e & 3))) & 0xFFu;
      if (byte & 0x80u) neg |= 1u << e;
    }
  }
  const int nwaves = gridDim.x * kHadWaves;
  const int per = (total_new + nwaves - 1) / nwaves;
  const int w0 = min(total_new, (int)(blockIdx.x * kHadWaves + wave) * per);
  const int w1 = min(total_new, w0 + per);
  if (w0 >= w1) return;
  // row slot q: rows [n0, n1), quarter q of [w0, w1)
  const int qper = (w1 - w0 + 3) / 4;
  const int n0 = min(w1, w0 + q * qper), n1 = min(w1, n0 + qper);
  const int gi = l >> 2;
  double* bd = sm.d[wave][q];
  float* bf = sm.f[wave][q];

  // Loads are unconditional: a row past the slot's end (or of an empty slot) loads row w0,
  // which is never stored.
  auto load_row = [&](int n) -> uint4 {
    const int nn = n < n1 ? n : w0;
    return *reinterpret_cast<const uint4*>(src + ((size_t)nn * g.hkv + h) * kHeadDim + 8 * l);
  };
  int seq = 0, first = 0, next_first = 0, sp = 0, slot = 0;
  if (n0 < n1) {
    seq = row_to_seq(new_offsets, batch, n0);
    first = new_offsets[seq];
    next_first = new_offsets[seq + 1];
    sp = start_pos[seq];
    slot = slot_ids ? slot_ids[seq] : seq;
  }
  int lp_cached = -1, page = -1, page_ahead = -1;
  uint4 cur[kHadAhead], nxt[kHadAhead];
#pragma unroll
  for (int u = 0; u < kHadAhead; ++u) cur[u] = load_row(n0 + u);
  for (int k = 0; k < qper; k += kHadAhead) {
#pragma unroll
    for (int u = 0; u < kHadAhead; ++u) nxt[u] = load_row(n0 + k + kHadAhead + u);
#pragma unroll
    for (int u = 0; u < kHadAhead; ++u) {
      const int n = n0 + k + u;
      const bool act = n < n1;  // uniform over the row slot
      // fp64 transform of the signed row; every lane computes (an inactive slot on row w0)
      const uint32_t xs[4] = {cur[u].x, cur[u].y, cur[u].z, cur[u].w};
      double v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const double x = (double)((e & 1) ? bf16_hi(xs[e >> 1]) : bf16_lo(xs[e >> 1]));
        v[e] = ((neg >> e) & 1u) ? -x : x;
      }
      // h = 1, 2, 4 in layout A
      fwht_pair(v[0], v[1]); fwht_pair(v[2], v[3]); fwht_pair(v[4], v[5]); fwht_pair(v[6], v[7]);
      fwht_pair(v[0], v[2]); fwht_pair(v[1], v[3]); fwht_pair(v[4], v[6]); fwht_pair(v[5], v[7]);
      fwht_pair(v[0], v[4]); fwht_pair(v[1], v[5]); fwht_pair(v[2], v[6]); fwht_pair(v[3], v[7]);
      // to layout B
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *reinterpret_cast<double2*>(bd + 8 * l + 2 * j) = make_double2(v[2 * j], v[2 * j + 1]);
      wave_lds_sync();
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = bd[l + 16 * e];
      wave_lds_sync();
      // h = 8: the lower lane of (l, l ^ 8) takes lower + upper, the upper lower - upper
      const uint32_t sign8 = (l & 8) ? 0x80000000u : 0u;
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = lane_xor_f64<8>(v[e]) + with_sign(v[e], sign8);
      // h = 16, 32, 64 in layout B (channel l + 16e)
      fwht_pair(v[0], v[1]); fwht_pair(v[2], v[3]); fwht_pair(v[4], v[5]); fwht_pair(v[6], v[7]);
      fwht_pair(v[0], v[2]); fwht_pair(v[1], v[3]); fwht_pair(v[4], v[6]); fwht_pair(v[5], v[7]);
      fwht_pair(v[0], v[4]); fwht_pair(v[1], v[5]); fwht_pair(v[2], v[6]); fwht_pair(v[3], v[7]);
      // scale, round to fp32, back to layout A
#pragma unroll
      for (int e = 0; e < 8; ++e) bf[l + 16 * e] = (float)(v[e] * kHadScale);
      wave_lds_sync();
      float y[8];
      {
        const float4 y0 = *reinterpret_cast<const float4*>(bf + 8 * l);
        const float4 y1 = *reinterpret_cast<const float4*>(bf + 8 * l + 4);
        y[0] = y0.x; y[1] = y0.y; y[2] = y0.z; y[3] = y0.w;
        y[4] = y1.x; y[5] = y1.y; y[6] = y1.z; y[7] = y1.w;
      }
      wave_lds_sync();

      // group extremes over the group's 4 lanes, scale/zero, codes
      float mx = y[0], mn = y[0];
#pragma unroll
      for (int e = 1; e < 8; ++e) {
        mx = fmaxf(mx, y[e]);
        mn = fminf(mn, y[e]);
      }
      mx = fmaxf(mx, lane_xor_f32<1>(mx));
      mn = fminf(mn, lane_xor_f32<1>(mn));
      mx = fmaxf(mx, lane_xor_f32<2>(mx));
      mn = fminf(mn, lane_xor_f32<2>(mn));
      _Float16 s16, z16;
      group_params(mx, mn, clip, s16, z16);
      const float sc = (float)s16, z = (float)z16;
      uint32_t code[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) code[e] = (uint32_t)code_of(y[e], sc, z);
      // code words: K word d = l / 2 (lanes 2d, 2d + 1; channel 16d + c at bits
      // 8 (c / 4) + 2 (c % 4)); V halves r16 = 8 (l % 2) + e of the lanes of one parity, channel
      // r16 + 16 nb at bits 2 nb (nb = l / 2), two halves per word
      uint32_t kw = 0;
      uint32_t hv[4];
      if (!is_v) {
#pragma unroll
        for (int e = 0; e < 8; ++e) kw |= code[e] << (8 * (e >> 2) + 2 * (e & 3));
        kw <<= 16 * (l & 1);
        kw |= lane_xor<1>(kw);
      } else {
        const int nb = l >> 1;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          uint32_t w = (code[2 * j] << (2 * nb)) | (code[2 * j + 1] << (16 + 2 * nb));
          w |= lane_xor<2>(w);
          w |= lane_xor<4>(w);
          w |= lane_xor<8>(w);
          hv[j] = w;
        }
      }

      // placement of the slot's row
      RowInfo info{-1, 0, -1};
      if (act) {
        if (n >= next_first) {   // the row starts a later sequence (rows are consecutive)
          seq = advance_seq(new_offsets, batch, seq + 1, n);
          first = new_offsets[seq];
          next_first = new_offsets[seq + 1];
          sp = start_pos[seq];
          slot = slot_ids ? slot_ids[seq] : seq;
          lp_cached = -1;
          page_ahead = -1;
        }
        const int pos = sp + (n - first);
        const int new_len = sp + (next_first - first);
        const int lp = pos / kPage;
        if (lp != lp_cached) {
          page = (lp == lp_cached + 1 && lp_cached >= 0) ? page_ahead
                 : ((pos >= 0 && lp < g.max_pages) ? block_table[(size_t)seq * g.max_pages + lp] : -1);
          lp_cached = lp;
          page_ahead = (pos >= 0 && lp + 1 < g.max_pages) ? block_table[(size_t)seq * g.max_pages + lp + 1]
                                                         : -1;
        }
        if (pos >= 0 && page >= 0 && page < g.num_pages && lp < g.max_pages) {
          info.rec = ((long long)page * g.hkv + h) * kRecord;
          info.slot_in_page = pos % kPage;
        }
        int row = -1;
        if (pos >= 0 && pos < g.num_sink) row = pos;
        else if (g.window > 0 && pos >= g.num_sink && pos >= new_len - g.window)
          row = g.num_sink + pos % g.window;
        if (row >= 0 && sinkwin != nullptr && slot >= 0 && slot < g.num_slots)
          info.sw = (((long long)slot * g.hkv + h) * (g.num_sink + g.window) + row) * 2 * kHeadDim +
                    (is_v ? kHeadDim : 0);
      }
      if (info.rec >= 0) {
        const int sl = info.slot_in_page;
        if ((l & 3) == 0) store_meta(pages, info, is_v, gi, meta_word(s16, z16));
        if (!is_v) {
          if ((l & 1) == 0) {
            const int d = l >> 1;
            *reinterpret_cast<uint32_t*>(pages + info.rec + kKCodes + 8 * (16 * (d % 4) + sl) +
                                         4 * (d / 4)) = kw;
          }
        } else {
          // lane l stores half r16 = 8 (l % 2) + l / 2
          const int idx = l >> 1, jj = idx >> 1;
          const uint32_t w = jj == 0 ? hv[0] : jj == 1 ? hv[1] : jj == 2 ? hv[2] : hv[3];
          const int r16 = 8 * (l & 1) + idx;
          uint8_t* base = pages + info.rec + kVCodes + 4 * ((sl % 4) / 2) + 2 * (sl % 2);
          *reinterpret_cast<uint16_t*>(base + 8 * (16 * (sl / 4) + r16)) =
              (uint16_t)(w >> (16 * (idx & 1)));
        }
      }
      if (info.sw >= 0) {
        uint4 o;
        o.x = (uint32_t)f32_to_bf16_rne(y[0]) | ((uint32_t)f32_to_bf16_rne(y[1]) << 16);
        o.y = (uint32_t)f32_to_bf16_rne(y[2]) | ((uint32_t)f32_to_bf16_rne(y[3]) << 16);
        o.z = (uint32_t)f32_to_bf16_rne(y[4]) | ((uint32_t)f32_to_bf16_rne(y[5]) << 16);
        o.w = (uint32_t)f32_to_bf16_rne(y[6]) | ((uint32_t)f32_to_bf16_rne(y[7]) << 16);
        *reinterpret_cast<uint4*>(sinkwin + info.sw + 8 * l) = o;
      }
    }
#pragma unroll
    for (int u = 0; u < kHadAhead; ++u) cur[u] = nxt[u];
  }
}

}  // namespace

hipError_t launch_append_hadamard(const CacheGeom& g, uint8_t* pages, uint16_t* sinkwin,
                                  const int32_t* block_table, const int32_t* slot_ids, int batch,
                                  int total_new, const uint16_t* k_new, const uint16_t* v_new,
                                  const int32_t* new_offsets, const int32_t* start_pos,
                                  const int8_t* signs_k, const int8_t* signs_v, float clip_k,
                                  float clip_v, hipStream_t stream) {
  if (batch == 0 || total_new == 0) return hipSuccess;
  int cus = current_device_cus();
  if (cus <= 0) cus = 256;
  // about 16 waves per SIMD over the 2 * Hkv (head, K|V) pairs; at least one row per wave
  const int want = max(1, 64 * cus / (2 * g.hkv * kHadWaves));
  const int blocks = max(1, min(want, (total_new + kHadWaves - 1) / kHadWaves));
  hipLaunchKernelGGL(rotate_quantize_hadamard_kernel, dim3(blocks, g.hkv, 2), dim3(64 * kHadWaves),
                     0, stream, g, pages, sinkwin, block_table, slot_ids, batch, total_new, k_new,
                     v_new, new_offsets, start_pos, signs_k, signs_v, clip_k, clip_v);
  return hipGetLastError();
}

hipError_t launch_append(const CacheGeom& g, uint8_t* pages, uint16_t* sinkwin,
                         const int32_t* block_table, const int32_t* slot_ids, int batch,
                         int total_new, const uint16_t* k_new, const uint16_t* v_new,
                         const int32_t* new_offsets, const int32_t* start_pos,
                         const float* rot_k, const float* rot_v, const float* k_mean,
                         float clip_k, float clip_v, int method, hipStream_t stream) {
  if (batch == 0 || total_new == 0) return hipSuccess;
  if (method == kAppendAuto) method = total_new >= kMatrixAppendRows ? kAppendMatrix : kAppendVector;
  if (method == kAppendMatrix) {
    int cus = current_device_cus();
    if (cus <= 0) cus = 256;
    // two resident workgroups per CU (R^T takes most of their LDS) over the 2 * Hkv (KV head,
    // K|V) pairs.  A V block costs ~15% more than a K block (its waves exchange code pairs
    // behind a barrier), so K gets 15 of every 32 workgroups of a head; centered keys leave
    // more values uncertain (about 1.8% against 1.2% recomputed), so with a key mean K gets 19.
    const int tiles = (total_new + kMBlock - 1) / kMBlock;
    const int per_head = 2 * max(1, min(tiles, (2 * cus + 2 * g.hkv - 1) / (2 * g.hkv)));
    const int k_share = k_mean != nullptr ? 19 : 15;
    const int k_groups = max(1, min(per_head - 1, (per_head * k_share + 16) / 32));
    hipLaunchKernelGGL(rotate_quantize_prefill_kernel<2>, dim3(per_head, g.hkv), dim3(kMThreads), 0,
                       stream, g, pages, sinkwin, block_table, slot_ids, batch, total_new, k_new,
                       v_new, new_offsets, start_pos, rot_k, rot_v, k_mean, clip_k, clip_v,
                       k_groups);
    return hipGetLastError();
  }
  // few rows: 4 per workgroup, so that the launch covers more CUs
  if (total_new <= 64 * 16) {
    dim3 grid((total_new + 3) / 4, g.hkv, 2);
    hipLaunchKernelGGL(rotate_quantize_append_kernel<4>, grid, dim3(kAppendThreads), 0, stream, g, pages,
                       sinkwin, block_table, slot_ids, batch, total_new, k_new, v_new, new_offsets,
                       start_pos, rot_k, rot_v, k_mean, clip_k, clip_v);
  } else {
    dim3 grid((total_new + 15) / 16, g.hkv, 2);
    hipLaunchKernelGGL(rotate_quantize_append_kernel<16>, grid, dim3(kAppendThreads), 0, stream, g, pages,
                       sinkwin, block_table, slot_ids, batch, total_new, k_new, v_new, new_offsets,
                       start_pos, rot_k, rot_v, k_mean, clip_k, clip_v);
  }
  return hipGetLastError();
}

hipError_t launch_prefill_int4(const CacheGeom& g, uint8_t* pages, uint16_t* sinkwin,
                               const int32_t* block_table, const int32_t* slot_ids, int batch,
                               int total_new, const uint16_t* k_new, const uint16_t* v_new,
                               const int32_t* new_offsets, const int32_t* start_pos,
                               const float* rot_k, const float* rot_v, const float* k_mean,
                               float clip_k, float clip_v, hipStream_t stream) {
  if (batch == 0 || total_new == 0) return hipSuccess;
  int cus = current_device_cus();
  if (cus <= 0) cus = 256;
  // as the INT2 form; INT4 V blocks need no exchange between groups, so K and V blocks cost
  // about the same: half of the workgroups each (19 of 32 for centered keys)
  const int tiles = (total_new + kMBlock - 1) / kMBlock;
  const int per_head = 2 * max(1, min(tiles, (2 * cus + 2 * g.hkv - 1) / (2 * g.hkv)));
  const int k_share = k_mean != nullptr ? 19 : 16;
  const int k_groups = max(1, min(per_head - 1, (per_head * k_share + 16) / 32));
  hipLaunchKernelGGL(rotate_quantize_prefill_kernel<4>, dim3(per_head, g.hkv), dim3(kMThreads), 0,
                     stream, g, pages, sinkwin, block_table, slot_ids, batch, total_new, k_new,
                     v_new, new_offsets, start_pos, rot_k, rot_v, k_mean, clip_k, clip_v, k_groups);
  return hipGetLastError();
}

}  // namespace oscar
