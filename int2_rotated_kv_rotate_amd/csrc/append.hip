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
// A workgroup of 8 waves serves one (KV head, K|V) and loops over 64-row tiles.  Wave w owns
// output channels 16w .. 16w+15: its A operands are the rows of R^T for those channels, split
// exactly into three bf16 pieces (R = p0 + p1 + p2: 24 significand bits in three 8-bit pieces)
// and held in registers for the whole loop.  The B operand is the bf16 input rows (exact) from
// LDS.  For each 32-channel slice s of the input, three v_mfma_f32_16x16x32_bf16 accumulate
// p2, p1 and p0 (small pieces first) into a slice accumulator, and y = (a0 + a1) + (a2 + a3).
//
// Error bound.  The products are exact.  Measured on gfx950, one such instruction runs four
// passes over its 8-product blocks; a pass adds its products, aligned to the largest of them
// (bits below 2^-24 of it dropped), to the accumulator with one fp32 round-to-nearest.  Per
// slice that is at most 7u sum|terms| of dropped bits (u = 2^-24) and, since the small pieces
// come first, about 4.1u sum|terms| of rounding; the two levels of fp32 additions and the
// defined value's own rounding to fp32 add 3u.  So |y_mc - y| <= 14.1 u sum_i |x_i R_ij| <=
// 14.1 u ||x|| ||R_.j||.  The kernel takes E = 64 u ||x|| ||R_.j|| plus 2^-100 for flushed
// subnormals, computed 5% high so that y -+ E rounded to nearest still encloses [y - E, y + E].
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
// Recomputation reads R (fp32) from LDS, where the workgroup stages it once; four lanes share a
// value and the midpoint argument below keeps the result the defined one.
constexpr int kPTile = 64;
constexpr int kPThreads = 512;
constexpr int kXStride = kHeadDim + 8;   // bf16 per LDS row of x: 16-byte rows, skewed banks
constexpr int kYStride = kHeadDim + 4;   // floats per LDS row of y
constexpr int kExact = 0x80;             // s_code mark: s_y holds the defined value
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

constexpr int kRStride = kHeadDim + 1;   // floats per LDS row of R: column reads spread banks
constexpr int kListCap = kPTile * kHeadDim;

// Recompute the listed (row, channel) values as defined, four lanes per value: lane q sums the
// products of inputs 32q .. 32q+31 in fp64, and the four partial sums are combined.  That sum
// differs from the defined ascending one by at most 2 * 127 * 2^-53 sum|terms| <= 2^-45 ||x||
// ||R_.c||, and after the fp64 subtraction of the key-mean term C_c (0 without a mean) by at
// most that plus two fp64 ulps.  Unless it lies that close to a midpoint between fp32 values or
// to zero (where the sign of a zero result is decided), both round to the same fp32 value, and
// the rare value that close is summed again in ascending order.  `pass2` also recodes the
// values (the defined formula); otherwise they are marked exact.
// Called by all threads of the workgroup.
__device__ void recompute_listed(const uint16_t* __restrict__ list, int n,
                                 const float (*s_rot)[kRStride], const uint16_t (*s_x)[kXStride],
                                 const double* s_cd, const float* s_nrm, const float* s_cng,
                                 float (*s_y)[kYStride], uint8_t (*s_code)[kHeadDim],
                                 const float2 (*s_sz)[kGroups], bool pass2) {
  const int t = threadIdx.x, q = t & 3;
  for (int k0 = 0; k0 < n; k0 += kPThreads / 4) {
    const int k = k0 + (t >> 2);
    const bool act = k < n;
    const int it = act ? list[k] : 0;
    const int r = it / kHeadDim, c = it % kHeadDim;
    double part = 0.0;
    if (act) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint4 xv = *reinterpret_cast<const uint4*>(&s_x[r][32 * q + 8 * j]);
        const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x = e & 1 ? bf16_hi(xw[e / 2]) : bf16_lo(xw[e / 2]);
          part = __fma_rn((double)x, (double)s_rot[32 * q + 8 * j + e][c], part);
        }
      }
    }
    part += __shfl_xor(part, 1);
    part += __shfl_xor(part, 2);
    if (act && q == 0) {
      const double v = part - s_cd[c];
      float f = (float)v;
      const double tol = (double)s_nrm[r] * (double)s_cng[c / kGroup] * 0x1p-44 + fabs(v) * 0x1p-50;
      const double m_lo = ((double)f + (double)down(f)) * 0.5;
      const double m_hi = ((double)f + (double)up(f)) * 0.5;
      if (fabs(v - m_lo) <= tol || fabs(v - m_hi) <= tol || fabs(v) <= tol) {
        double acc = 0.0;
        for (int i = 0; i < kHeadDim; ++i)
          acc = __fma_rn((double)bf16_to_f32(s_x[r][i]), (double)s_rot[i][c], acc);
        f = (float)(acc - s_cd[c]);
      }
      s_y[r][c] = f;
      const float2 sz = s_sz[r][c / kGroup];
      s_code[r][c] = pass2 ? (uint8_t)code_of(f, sz.x, sz.y) : (uint8_t)kExact;
    }
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

__global__ __launch_bounds__(kPThreads, 2) void rotate_quantize_prefill_kernel(
    CacheGeom g, uint8_t* __restrict__ pages, uint16_t* __restrict__ sinkwin,
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ slot_ids, int batch,
    int total_new, const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
    const int32_t* __restrict__ new_offsets, const int32_t* __restrict__ start_pos,
    const float* __restrict__ rot_k, const float* __restrict__ rot_v,
    const float* __restrict__ k_mean, float clip_k, float clip_v, int k_groups) {
#pragma clang fp contract(off)
  __shared__ float s_rot[kHeadDim][kRStride];  // R (fp32), for the A operands and recomputation
  __shared__ __attribute__((aligned(16))) uint16_t s_x[kPTile][kXStride];
  __shared__ __attribute__((aligned(16))) float s_y[kPTile][kYStride];
  __shared__ __attribute__((aligned(16))) uint8_t s_code[kPTile][kHeadDim];
  __shared__ float2 s_sz[kPTile][kGroups];     // (scale, zero) of each group, fp32
  __shared__ uint16_t s_list[kListCap];        // (row, channel) to recompute: 128 r + c
  __shared__ RowInfo s_info[kPTile];
  __shared__ float s_err[kPTile];              // 64 u ||x|| per row, 5% high
  __shared__ float s_nrm[kPTile];              // ||x|| per row (rounded up)
  __shared__ float s_cng[kGroups];             // the largest ||R_.j|| of each group (rounded up)
  __shared__ float s_mu[kHeadDim];             // key mean (centered K only)
  __shared__ double s_cd[kHeadDim];            // C = mu . R (fp64; 0 without a mean)
  __shared__ __attribute__((aligned(16))) float s_cf[kHeadDim];  // fp32(C)
  __shared__ float s_cmax[kGroups];            // the largest |fp32(C_j)| of each group
  __shared__ int s_n[2];                       // list lengths of the two passes

  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int h = blockIdx.y;
  // workgroups [0, k_groups) of a KV head serve its K rows, the rest its V rows; x0 is this
  // workgroup's index among the G of its (head, K|V) pair
  const bool is_v = (int)blockIdx.x >= k_groups;
  const int G = is_v ? (int)gridDim.x - k_groups : k_groups;
  const int x0 = is_v ? (int)blockIdx.x - k_groups : (int)blockIdx.x;
  const float* rot = (is_v ? rot_v : rot_k) + (size_t)h * kHeadDim * kHeadDim;
  const uint16_t* src = is_v ? v_new : k_new;
  const float clip = is_v ? clip_v : clip_k;
  const int m = lane & 15, kq = lane >> 4;
  const bool centered = !is_v && k_mean != nullptr;
  if (centered && t < kHeadDim) s_mu[t] = k_mean[(size_t)h * kHeadDim + t];

  // Stage R: all 8 float4 loads of a thread first, then the (unaligned-row) LDS stores.
  {
    constexpr int kPer = kHeadDim * kHeadDim / 4 / kPThreads;  // 8
    const float4* rot4 = reinterpret_cast<const float4*>(rot);
    float4 rr[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) rr[k] = rot4[t + kPThreads * k];
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int e = 4 * (t + kPThreads * k), i = e / kHeadDim, j = e % kHeadDim;
      s_rot[i][j] = rr[k].x;
      s_rot[i][j + 1] = rr[k].y;
      s_rot[i][j + 2] = rr[k].z;
      s_rot[i][j + 3] = rr[k].w;
    }
  }
  __syncthreads();
  if (t < kHeadDim) {  // column norms (squared), parked in s_y before its first use
    float ss = 0.f;
    for (int i = 0; i < kHeadDim; ++i) ss = fmaf(s_rot[i][t], s_rot[i][t], ss);
    s_y[0][t] = ss;
    // key mean: C_t = sum_i mu_i R_it, fp64, i ascending (exact products)
    double cd = 0.0;
    if (centered)
      for (int i = 0; i < kHeadDim; ++i) cd = __fma_rn((double)s_mu[i], (double)s_rot[i][t], cd);
    s_cd[t] = cd;
    s_cf[t] = (float)cd;
  }
  __syncthreads();
  if (t < kGroups) {   // the largest per group, rounded up
    float cm = 0.f, cc = 0.f;
    for (int c = kGroup * t; c < kGroup * (t + 1); ++c) {
      cm = fmaxf(cm, s_y[0][c]);
      cc = fmaxf(cc, fabsf(s_cf[c]));
    }
    s_cng[t] = __builtin_sqrtf(cm) * 1.001f;
    s_cmax[t] = cc;
  }
  __syncthreads();
  // fp32(C) of this lane's four output channels (16w + 4kq + i), subtracted from the matrix-core
  // sums; 0 without a mean
  const float4 cfl = *reinterpret_cast<const float4*>(&s_cf[16 * wave + 4 * kq]);

  // A operands: lane (m, kq), slice s holds R[32s + 8kq + e][16w + m], e = 0..7, as 3 pieces.
  v8bf ra[4][3];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    uint16_t pc[3][8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float r0 = s_rot[32 * s + 8 * kq + e][16 * wave + m];
      pc[0][e] = f32_to_bf16_rne(r0);
      const float r1 = r0 - bf16_to_f32(pc[0][e]);
      pc[1][e] = f32_to_bf16_rne(r1);
      pc[2][e] = f32_to_bf16_rne(r1 - bf16_to_f32(pc[1][e]));
    }
#pragma unroll
    for (int q = 0; q < 3; ++q) {
      uint4 w;
      w.x = pc[q][0] | ((uint32_t)pc[q][1] << 16);
      w.y = pc[q][2] | ((uint32_t)pc[q][3] << 16);
      w.z = pc[q][4] | ((uint32_t)pc[q][5] << 16);
      w.w = pc[q][6] | ((uint32_t)pc[q][7] << 16);
      ra[s][q] = __builtin_bit_cast(v8bf, w);
    }
  }

  const int ntiles = (total_new + kPTile - 1) / kPTile;
  const bool has_store = sinkwin != nullptr;

  // Software pipeline over the tiles: while tile k is processed, its successor's input rows are
  // in flight into registers, and threads t < 64 look up the successor's row placements in
  // stages (one dependent load per stage, each consumed a phase later).
  auto load_rows = [&](int tl, uint4& a0, uint4& a1) {
    const int r = t >> 3, q = t & 7, n = tl * kPTile + r;
    a0 = uint4{0, 0, 0, 0};
    a1 = uint4{0, 0, 0, 0};
    if (tl < ntiles && n < total_new) {
      const uint4* rp = reinterpret_cast<const uint4*>(src + ((size_t)n * g.hkv + h) * kHeadDim);
      a0 = rp[q];
      a1 = rp[q + 8];
    }
  };
  uint4 u0, u1;
  load_rows(x0, u0, u1);
  int seq = 0;                         // sequence of this thread's row (t < 64)
  RowInfo info_next{-1, 0, -1};
  if (t < kPTile && x0 < ntiles && x0 * kPTile + t < total_new) {
    seq = row_to_seq(new_offsets, batch, x0 * kPTile + t);
    info_next = row_info(g, block_table, slot_ids, batch, new_offsets, start_pos, has_store,
                         x0 * kPTile + t, h, is_v);
  }

  // Round k takes tile k * G + (x + k) mod G (G workgroups per pair, x this one), one tile of
  // each block of G; the rotation spreads tiles that cost more (e.g. the last rows of every
  // sequence, whose BF16 copies are certified too) over all workgroups.  Successive tiles of a
  // workgroup increase, as the placement look-ahead needs.
  auto tile_of = [&](int k) { return k * G + (x0 + k) % G; };   // tile_of(0) == x0
  for (int k = 0, tile = x0; tile < ntiles; ++k, tile = tile_of(k)) {
    const int row0 = tile * kPTile;
    const int nrows = min(kPTile, total_new - row0);
    const int nt = tile_of(k + 1);     // the successor tile
    const int n_next = nt * kPTile + t;
    const bool look = t < kPTile && nt < ntiles && n_next < total_new;

    // Input rows into LDS (8 threads per row, 2 x 16 bytes each), their norms, placements.
    {
      const int r = t >> 3, q = t & 7;
      *reinterpret_cast<uint4*>(&s_x[r][8 * q]) = u0;
      *reinterpret_cast<uint4*>(&s_x[r][8 * q + 64]) = u1;
      const uint32_t xw[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
      double ss = 0.0;   // fp64: no underflow for rows of subnormal values
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        ss = __fma_rn((double)bf16_lo(xw[k]), (double)bf16_lo(xw[k]), ss);
        ss = __fma_rn((double)bf16_hi(xw[k]), (double)bf16_hi(xw[k]), ss);
      }
      ss += __shfl_xor(ss, 1);
      ss += __shfl_xor(ss, 2);
      ss += __shfl_xor(ss, 4);
      if (q == 0) {
        const float nrm = (float)__builtin_sqrt(ss) * (1.0f + 0x1p-20f);
        s_nrm[r] = nrm;
        s_err[r] = kErrScale * nrm;
      }
      if (t < kPTile) s_info[t] = info_next;
      if (t == 0) s_n[0] = s_n[1] = 0;
    }
    load_rows(nt, u0, u1);
    // placement stage 1: is the successor's row still in the same sequence?
    int off_up = 0;
    if (look && seq + 1 < batch) off_up = new_offsets[seq + 1];
    __syncthreads();

    // y on the matrix cores: channels 16w .. 16w+15 of the tile's 64 rows.
#pragma unroll 1
    for (int tt = 0; tt < kPTile / 16; ++tt) {
      const uint16_t* xr = &s_x[16 * tt + m][8 * kq];
      v4f acc[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const v8bf xb = __builtin_bit_cast(v8bf, *reinterpret_cast<const uint4*>(xr + 32 * s));
        acc[s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ra[s][2], xb, v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
        acc[s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ra[s][1], xb, acc[s], 0, 0, 0);
        acc[s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ra[s][0], xb, acc[s], 0, 0, 0);
      }
      float4 y;
      y.x = ((acc[0][0] + acc[1][0]) + (acc[2][0] + acc[3][0])) - cfl.x;
      y.y = ((acc[0][1] + acc[1][1]) + (acc[2][1] + acc[3][1])) - cfl.y;
      y.z = ((acc[0][2] + acc[1][2]) + (acc[2][2] + acc[3][2])) - cfl.z;
      y.w = ((acc[0][3] + acc[1][3]) + (acc[2][3] + acc[3][3])) - cfl.w;
      // D row = channel 16w + 4kq + i, column = token 16tt + m
      *reinterpret_cast<float4*>(&s_y[16 * tt + m][16 * wave + 4 * kq]) = y;
    }
    __syncthreads();

    // placement stage 2: the successor row's sequence, then its per-sequence values
    int first = 0, next_first = 0, sp = 0, slot = 0;
    if (look) {
      if (seq + 1 < batch && off_up <= n_next) seq = advance_seq(new_offsets, batch, seq + 1, n_next);
      first = new_offsets[seq];
      next_first = new_offsets[seq + 1];
      sp = start_pos[seq];
      slot = slot_ids ? slot_ids[seq] : seq;
    }

    // Thread -> (row r, group gi, half of the group's 32 channels) for the group passes.
    const int r = t >> 3, gi = (t >> 1) & 3, half = t & 1;
    const int c0 = gi * kGroup + 16 * half;
    const float er = s_err[r];

    // Pass 1: certify each group's scale and zero; if they are not certain, flag every channel
    // that can hold the group's maximum or minimum.
    {
      float yv[16];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float4 a = *reinterpret_cast<const float4*>(&s_y[r][c0 + 4 * k]);
        yv[4 * k] = a.x; yv[4 * k + 1] = a.y; yv[4 * k + 2] = a.z; yv[4 * k + 3] = a.w;
      }
      float mx = yv[0], mn = yv[0];
#pragma unroll
      for (int c = 1; c < 16; ++c) {
        mx = fmaxf(mx, yv[c]);
        mn = fminf(mn, yv[c]);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 1));
      mn = fminf(mn, __shfl_xor(mn, 1));
      const float E = er * s_cng[gi] + kErrAbs +
                      (centered ? (s_cmax[gi] + 2.0f * fmaxf(fabsf(mx), fabsf(mn))) * 0x1p-22f : 0.0f);
      _Float16 s_hi, z_hi, s_lo, z_lo;
      group_params(mx + E, mn - E, clip, s_hi, z_lo);
      group_params(mx - E, mn + E, clip, s_lo, z_hi);
      const bool sure = __builtin_bit_cast(uint16_t, s_hi) == __builtin_bit_cast(uint16_t, s_lo) &&
                        __builtin_bit_cast(uint16_t, z_hi) == __builtin_bit_cast(uint16_t, z_lo);
      *reinterpret_cast<uint4*>(&s_code[r][c0]) = uint4{0, 0, 0, 0};
      if (!sure && r < nrows) {
        const float top = mx - 2.0f * E, bot = mn + 2.0f * E;
#pragma unroll
        for (int c = 0; c < 16; ++c)
          if (yv[c] >= top || yv[c] <= bot) s_list[atomicAdd(&s_n[0], 1)] = (uint16_t)(kHeadDim * r + c0 + c);
      }
    }
    __syncthreads();
    recompute_listed(s_list, s_n[0], s_rot, s_x, s_cd, s_nrm, s_cng, s_y, s_code, s_sz, false);
    __syncthreads();

    // placement stage 3: page of the successor row
    int pos = 0, page = -1;
    if (look) {
      pos = sp + (n_next - first);
      const int lp = pos / kPage;
      if (pos >= 0 && lp < g.max_pages) page = block_table[(size_t)seq * g.max_pages + lp];
    }

    // Pass 2: the group's scale and zero (now the defined ones), every code and BF16 copy; flag
    // what the bound cannot certify (E taken for the group's largest column norm).
    {
      float mx, mn;
      {
        const float4 a = *reinterpret_cast<const float4*>(&s_y[r][c0]);
        mx = fmaxf(fmaxf(a.x, a.y), fmaxf(a.z, a.w));
        mn = fminf(fminf(a.x, a.y), fminf(a.z, a.w));
      }
#pragma unroll
      for (int k = 1; k < 4; ++k) {
        const float4 a = *reinterpret_cast<const float4*>(&s_y[r][c0 + 4 * k]);
        mx = fmaxf(mx, fmaxf(fmaxf(a.x, a.y), fmaxf(a.z, a.w)));
        mn = fminf(mn, fminf(fminf(a.x, a.y), fminf(a.z, a.w)));
      }
      mx = fmaxf(mx, __shfl_xor(mx, 1));
      mn = fminf(mn, __shfl_xor(mn, 1));
      _Float16 s16, z16;
      group_params(mx, mn, clip, s16, z16);
      const float sc = (float)s16, z = (float)z16;
      const float inv = sc != 0.0f ? 1.0f / sc : 0.0f;
      const RowInfo info = s_info[r];
      if (half == 0) {
        s_sz[r][gi] = make_float2(sc, z);
        if (r < nrows && info.rec >= 0) store_meta(pages, info, is_v, gi, meta_word(s16, z16));
      }
      const bool bf = info.sw >= 0;
      const float Eg = er * s_cng[gi] + kErrAbs +
                       (centered ? (s_cmax[gi] + 2.0f * fmaxf(fabsf(mx), fabsf(mn))) * 0x1p-22f : 0.0f);
      // code margins of the group (see above), taken at its largest |y| (>= every |y| in it):
      // one for values recomputed in pass 1 (E = 0), one for the others
      const float gabs = fmaxf(fabsf(mx), fabsf(mn)) + fabsf(z);
      const float mt_exact = (gabs * 0x1p-23f) * inv * 1.01f + 0x1p-19f;
      const float mt_bound = (Eg + (gabs + Eg) * 0x1p-23f) * inv * 1.01f + 0x1p-19f;
      const uint4 mk = *reinterpret_cast<const uint4*>(&s_code[r][c0]);
      const uint32_t mw[4] = {mk.x, mk.y, mk.z, mk.w};
      uint32_t cw[4] = {0, 0, 0, 0};
      unsigned flagged = 0;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float4 a = *reinterpret_cast<const float4*>(&s_y[r][c0 + 4 * k]);
        const float yk[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float y = yk[i];
          const bool exact = ((mw[k] >> (8 * i)) & 0xFF) == kExact;
          // t within mt of the defined t (see above); the code is certain when no boundary
          // 1/2, 3/2, 5/2 lies within mt of t.  The distance to the nearest half-integer is at
          // most the distance to those three, so comparing it is conservative.
          const float tq = (y - z) * inv;
          const float dist = fabsf(__builtin_amdgcn_fractf(tq) - 0.5f);
          bool ok = dist > (exact ? mt_exact : mt_bound);
          if (bf) {
            const float E = exact ? 0.0f : Eg;
            ok = ok && f32_to_bf16_rne(y - E) == f32_to_bf16_rne(y + E);
          }
          const int code = (int)fminf(fmaxf(__builtin_rintf(tq), 0.0f), 3.0f);
          cw[k] |= (uint32_t)code << (8 * i);
          flagged |= (ok ? 0u : 1u) << (4 * k + i);
        }
      }
      *reinterpret_cast<uint4*>(&s_code[r][c0]) = uint4{cw[0], cw[1], cw[2], cw[3]};
      if (r < nrows)
        while (flagged) {
          const int c = __builtin_ctz(flagged);
          flagged &= flagged - 1u;
          s_list[atomicAdd(&s_n[1], 1)] = (uint16_t)(kHeadDim * r + c0 + c);
        }
    }
    __syncthreads();
    recompute_listed(s_list, s_n[1], s_rot, s_x, s_cd, s_nrm, s_cng, s_y, s_code, s_sz, true);
    __syncthreads();

    // placement stage 4: the successor row's record and sink/window row
    if (look) {
      RowInfo info{-1, 0, -1};
      if (pos >= 0 && page >= 0 && page < g.num_pages && pos / kPage < g.max_pages) {
        info.rec = ((long long)page * g.hkv + h) * kRecord;
        info.slot_in_page = pos % kPage;
      }
      const int new_len = sp + (next_first - first);
      int row = -1;
      if (pos >= 0 && pos < g.num_sink) row = pos;
      else if (g.window > 0 && pos >= g.num_sink && pos >= new_len - g.window)
        row = g.num_sink + pos % g.window;
      if (row >= 0 && has_store && slot >= 0 && slot < g.num_slots)
        info.sw = (((long long)slot * g.hkv + h) * (g.num_sink + g.window) + row) * 2 * kHeadDim +
                  (is_v ? kHeadDim : 0);
      info_next = info;
    } else {
      info_next = RowInfo{-1, 0, -1};
    }

    // Pack the codes into the records; BF16 copies of sink/window rows.
    {
      const int q = t & 7;
      const RowInfo info = s_info[r];
      if (r < nrows && info.rec >= 0 && !is_v) {
        const uint4 cv = *reinterpret_cast<const uint4*>(&s_code[r][16 * q]);
        const uint32_t cwd[4] = {cv.x, cv.y, cv.z, cv.w};
        uint32_t w = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint32_t b = cwd[k];  // four codes, one per byte
          const uint32_t packed = (b & 3u) | ((b >> 6) & 0xCu) | ((b >> 12) & 0x30u) | ((b >> 18) & 0xC0u);
          w |= packed << (8 * k);
        }
        *reinterpret_cast<uint32_t*>(pages + info.rec + kKCodes +
                                     8 * (16 * (q % 4) + info.slot_in_page) + 4 * (q / 4)) = w;
      }
      if (r < nrows && info.sw >= 0) {
        uint32_t o[8];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float4 a = *reinterpret_cast<const float4*>(&s_y[r][16 * q + 4 * k]);
          o[2 * k] = f32_to_bf16_rne(a.x) | ((uint32_t)f32_to_bf16_rne(a.y) << 16);
          o[2 * k + 1] = f32_to_bf16_rne(a.z) | ((uint32_t)f32_to_bf16_rne(a.w) << 16);
        }
        uint4* dst = reinterpret_cast<uint4*>(sinkwin + info.sw + 16 * q);
        dst[0] = uint4{o[0], o[1], o[2], o[3]};
        dst[1] = uint4{o[4], o[5], o[6], o[7]};
      }
    }
    if (is_v) {
      for (int e = t; e < kPTile * 16; e += kPThreads) {
        const int rr = e >> 4, c16 = e & 15;
        const RowInfo info = s_info[rr];
        if (rr < nrows && info.rec >= 0) store_v_half(pages, info, s_code[rr], c16);
      }
    }
    __syncthreads();
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
// One wavefront per row at a time: lane l holds channels 2l and 2l + 1; stage h = 1 is inside
// the lane and stage h = 2m pairs lane l with lane l ^ m.  Each wave takes a contiguous range
// of rows (the row's sequence, page and slot advance incrementally, the next page id is read
// ahead) and loads the next kHadBatch rows while it computes the current ones.  Group g
// (channels 32g .. 32g + 31) is lanes 16g .. 16g + 15.

constexpr double kHadScale = 0x1.6a09e667f3bcdp-4;   // the double nearest to 2^-3.5 (sqrt(2)/16)

// One cross-lane FWHT stage h = 2M on the lane's two values.
template <int M>
__device__ __forceinline__ void fwht_stage(double& a, double& b, int lane) {
  const double pa = lane_xor_f64<M>(a), pb = lane_xor_f64<M>(b);
  const bool upper = (lane & M) != 0;   // lower: a + partner; upper: partner - a
  a = pa + (upper ? -a : a);
  b = pb + (upper ? -b : b);
}
constexpr int kHadWaves = 4;
constexpr int kHadBatch = 8;

__global__ __launch_bounds__(64 * kHadWaves) void rotate_quantize_hadamard_kernel(
    CacheGeom g, uint8_t* __restrict__ pages, uint16_t* __restrict__ sinkwin,
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ slot_ids, int batch,
    int total_new, const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
    const int32_t* __restrict__ new_offsets, const int32_t* __restrict__ start_pos,
    const int8_t* __restrict__ signs_k, const int8_t* __restrict__ signs_v, float clip_k,
    float clip_v) {
#pragma clang fp contract(off)
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h = blockIdx.y;
  const bool is_v = blockIdx.z != 0;
  const uint16_t* src = is_v ? v_new : k_new;
  const int8_t* sg = is_v ? signs_v : signs_k;
  const float clip = is_v ? clip_v : clip_k;
  const bool neg0 = sg != nullptr && sg[h * kHeadDim + 2 * lane] < 0;
  const bool neg1 = sg != nullptr && sg[h * kHeadDim + 2 * lane + 1] < 0;
  const int nwaves = gridDim.x * kHadWaves;
  const int per = (total_new + nwaves - 1) / nwaves;
  const int n0 = min(total_new, (int)(blockIdx.x * kHadWaves + wave) * per);
  const int n1 = min(total_new, n0 + per);
  if (n0 >= n1) return;
  const int gi = lane >> 4;

  auto load_row = [&](int n) -> uint32_t {
    return *reinterpret_cast<const uint32_t*>(src + ((size_t)n * g.hkv + h) * kHeadDim + 2 * lane);
  };
  int seq = row_to_seq(new_offsets, batch, n0);
  int first = new_offsets[seq], next_first = new_offsets[seq + 1];
  int sp = start_pos[seq];
  int slot = slot_ids ? slot_ids[seq] : seq;
  int lp_cached = -1, page = -1, page_ahead = -1;
  uint32_t cur[kHadBatch], nxt[kHadBatch];
#pragma unroll
  for (int u = 0; u < kHadBatch; ++u) cur[u] = n0 + u < n1 ? load_row(n0 + u) : 0u;
  for (int nb = n0; nb < n1; nb += kHadBatch) {
#pragma unroll
    for (int u = 0; u < kHadBatch; ++u) nxt[u] = nb + kHadBatch + u < n1 ? load_row(nb + kHadBatch + u) : 0u;
#pragma unroll 1
    for (int u = 0; u < kHadBatch; ++u) {
      const int n = nb + u;
      if (n >= n1) break;
      uint32_t xw = 0u;
#pragma unroll
      for (int k = 0; k < kHadBatch; ++k)
        if (k == u) xw = cur[k];
      if (n >= next_first) {   // the row starts a later sequence (rows are consecutive)
        seq = advance_seq(new_offsets, batch, seq + 1, n);
        first = new_offsets[seq];
        next_first = new_offsets[seq + 1];
        sp = start_pos[seq];
        slot = slot_ids ? slot_ids[seq] : seq;
        lp_cached = -1;
        page_ahead = -1;
      }
      // fp64 transform of the signed row
      double a = (double)bf16_lo(xw), b = (double)bf16_hi(xw);
      if (neg0) a = -a;
      if (neg1) b = -b;
      {
        const double s0 = a + b, d0 = a - b;
        a = s0;
        b = d0;
      }
      fwht_stage<1>(a, b, lane);
      fwht_stage<2>(a, b, lane);
      fwht_stage<4>(a, b, lane);
      fwht_stage<8>(a, b, lane);
      fwht_stage<16>(a, b, lane);
      fwht_stage<32>(a, b, lane);
      const float y0 = (float)(a * kHadScale), y1 = (float)(b * kHadScale);

      // group extremes over the 16 lanes of the group, scale/zero, codes
      float mx = fmaxf(y0, y1), mn = fminf(y0, y1);
      mx = fmaxf(mx, lane_xor_f32<1>(mx));
      mn = fminf(mn, lane_xor_f32<1>(mn));
      mx = fmaxf(mx, lane_xor_f32<2>(mx));
      mn = fminf(mn, lane_xor_f32<2>(mn));
      mx = fmaxf(mx, lane_xor_f32<4>(mx));
      mn = fminf(mn, lane_xor_f32<4>(mn));
      mx = fmaxf(mx, lane_xor_f32<8>(mx));
      mn = fminf(mn, lane_xor_f32<8>(mn));
      _Float16 s16, z16;
      group_params(mx, mn, clip, s16, z16);
      const float sc = (float)s16, z = (float)z16;
      const uint32_t c0 = (uint32_t)code_of(y0, sc, z), c1 = (uint32_t)code_of(y1, sc, z);

      // placement
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
      RowInfo info{-1, 0, -1};
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

      if (info.rec >= 0) {
        if ((lane & 15) == 0) store_meta(pages, info, is_v, gi, meta_word(s16, z16));
        const int sl = info.slot_in_page;
        if (!is_v) {
          // K word d = lane / 8 (channels 16d .. 16d + 15); channel 2l + e sits at byte
          // (l % 8) / 2, bits 2 * (2 * (l % 2) + e)
          const int sh = 8 * ((lane & 7) >> 1) + 4 * (lane & 1);
          uint32_t w = (c0 << sh) | (c1 << (sh + 2));
          w |= lane_xor<1>(w);
          w |= lane_xor<2>(w);
          w |= lane_xor<4>(w);
          if ((lane & 7) == 0) {
            const int d = lane >> 3;
            *reinterpret_cast<uint32_t*>(pages + info.rec + kKCodes + 8 * (16 * (d % 4) + sl) +
                                         4 * (d / 4)) = w;
          }
        } else {
          // V half of channel residue k = (2l + e) % 16 holds channel k + 16 nb at bits 2 nb,
          // nb = l / 8: lanes l % 8 == k / 2 combine
          uint32_t v0 = c0 << (2 * (lane >> 3)), v1 = c1 << (2 * (lane >> 3));
          v0 |= lane_xor<8>(v0);
          v1 |= lane_xor<8>(v1);
          v0 |= lane_xor<16>(v0);
          v1 |= lane_xor<16>(v1);
          v0 |= lane_xor<32>(v0);
          v1 |= lane_xor<32>(v1);
          if (lane < 8) {
            uint8_t* base = pages + info.rec + kVCodes + 4 * ((sl % 4) / 2) + 2 * (sl % 2);
            *reinterpret_cast<uint16_t*>(base + 8 * (16 * (sl / 4) + 2 * lane)) = (uint16_t)v0;
            *reinterpret_cast<uint16_t*>(base + 8 * (16 * (sl / 4) + 2 * lane + 1)) = (uint16_t)v1;
          }
        }
      }
      if (info.sw >= 0)
        *reinterpret_cast<uint32_t*>(sinkwin + info.sw + 2 * lane) =
            (uint32_t)f32_to_bf16_rne(y0) | ((uint32_t)f32_to_bf16_rne(y1) << 16);
    }
#pragma unroll
    for (int u = 0; u < kHadBatch; ++u) cur[u] = nxt[u];
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
  // about 8 waves per SIMD over the 2 * Hkv (head, K|V) pairs; at least one row per wave
  const int want = max(1, 32 * cus / (2 * g.hkv * kHadWaves));
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
    // one resident workgroup per CU (R and the tile take most of the LDS) over the 2 * Hkv
    // (KV head, K|V) pairs.  Centered keys leave more values uncertain (about 1.8% against
    // 1.2% recomputed), so with a key mean K gets 19 of every 32 workgroups of a head.
    const int tiles = (total_new + kPTile - 1) / kPTile;
    const int per_head = 2 * max(1, min(tiles, (cus + 2 * g.hkv - 1) / (2 * g.hkv)));
    const int k_groups = k_mean != nullptr ? max(1, min(per_head - 1, (per_head * 19 + 16) / 32))
                                           : per_head / 2;
    hipLaunchKernelGGL(rotate_quantize_prefill_kernel, dim3(per_head, g.hkv), dim3(kPThreads), 0,
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

}  // namespace oscar
