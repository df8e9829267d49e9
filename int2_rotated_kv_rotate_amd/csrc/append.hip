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

namespace oscar {
namespace {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kRows = 16;
constexpr int kThreads = 256;

// Keeps the compiler from fusing an fp32 result into a following conversion (it would
// otherwise turn fp16(c * mn) into one single-rounding mixed-precision FMA).
__device__ __forceinline__ float materialize(float x) {
  asm volatile("" : "+v"(x));
  return x;
}

struct RowInfo {
  long long rec;     // byte offset of the row's page record in the pool, -1 = skip
  int slot_in_page;  // 0..15
  long long sw;      // element offset of the row's bf16 K/V row in the store, -1 = none
};

// Where new row n (flattened over the batch) of KV head h goes.
__device__ RowInfo row_info(const CacheGeom& g, const int32_t* __restrict__ block_table,
                            const int32_t* __restrict__ slot_ids, int batch,
                            const int32_t* __restrict__ new_offsets,
                            const int32_t* __restrict__ start_pos, bool has_store, int n, int h,
                            bool is_v) {
  RowInfo info{-1, 0, -1};
  const int b = row_to_seq(new_offsets, batch, n);
  const int first = new_offsets[b];
  const int nnew = new_offsets[b + 1] - first;
  const int pos = start_pos[b] + (n - first);
  const int new_len = start_pos[b] + nnew;
  const int lp = pos / kPage;
  if (pos >= 0 && lp < g.max_pages) {
    const int page = block_table[(size_t)b * g.max_pages + lp];
    if (page >= 0 && page < g.num_pages) {
      info.rec = ((long long)page * g.hkv + h) * kRecord;
      info.slot_in_page = pos % kPage;
    }
  }
  const int slot = slot_ids ? slot_ids[b] : b;
  int row = -1;
  if (pos >= 0 && pos < g.num_sink) row = pos;
  else if (g.window > 0 && pos >= g.num_sink && pos >= new_len - g.window)
    row = g.num_sink + pos % g.window;
  if (row >= 0 && has_store && slot >= 0 && slot < g.num_slots)
    info.sw = (((long long)slot * g.hkv + h) * (g.num_sink + g.window) + row) * 2 * kHeadDim +
              (is_v ? kHeadDim : 0);
  return info;
}

// fp16 scale and zero of a group from its extremes: s = (c*mx - c*mn) / 3, z = c*mn, every
// step in fp32, a signed-zero extreme counting as +0.  Monotone: s never decreases with mx nor
// increases with mn, z never decreases with mn.
__device__ __forceinline__ void group_params(float mx, float mn, float clip, _Float16& s16,
                                             _Float16& z16) {
  mx = mx + 0.0f;
  mn = mn + 0.0f;
  const float mx_c = clip * mx;
  const float mn_c = clip * mn;
  const float width = mx_c - mn_c;
  const float s32 = width / 3.0f;
  s16 = (_Float16)materialize(s32);
  z16 = (_Float16)materialize(mn_c);
}

// clamp(rint((y - z) / s), 0, 3), 0 for a zero scale.  Monotone in y for s > 0.
__device__ __forceinline__ int code_of(float y, float s, float z) {
  if (s == 0.0f) return 0;
  float q = (y - z) / s;
  q = __builtin_rintf(q);
  q = fminf(fmaxf(q, 0.0f), 3.0f);
  return (int)q;
}

__device__ __forceinline__ uint32_t meta_word(_Float16 s16, _Float16 z16) {
  return (uint32_t)__builtin_bit_cast(uint16_t, s16) |
         ((uint32_t)__builtin_bit_cast(uint16_t, z16) << 16);
}

__device__ __forceinline__ void store_meta(uint8_t* pages, const RowInfo& info, bool is_v, int gi,
                                           uint32_t meta) {
  *reinterpret_cast<uint32_t*>(pages + info.rec + (is_v ? kVMeta : kKMeta) +
                               16 * info.slot_in_page + 4 * gi) = meta;
}

// K codes: 16-channel word d of a row -> dword at 8*(16*(d%4) + slot) + 4*(d/4), channel 16d+c
// at bits 8*(c/4) + 2*(c%4).
__device__ __forceinline__ void store_k_word(uint8_t* pages, const RowInfo& info,
                                             const uint8_t* codes, int d) {
  uint32_t w = 0;
  for (int c = 0; c < 16; ++c) w |= (uint32_t)codes[16 * d + c] << (8 * (c / 4) + 2 * (c % 4));
  *reinterpret_cast<uint32_t*>(pages + info.rec + kKCodes +
                               8 * (16 * (d % 4) + info.slot_in_page) + 4 * (d / 4)) = w;
}

// V codes: channel residue c16 of a row -> 16-bit half (slot%2) of dword (slot%4)/2 of chunk
// 16*(slot/4) + c16; channel c16 + 16*nb at bits 2*nb of the half.
__device__ __forceinline__ void store_v_half(uint8_t* pages, const RowInfo& info,
                                             const uint8_t* codes, int c16) {
  uint32_t hw = 0;
  for (int nb = 0; nb < 8; ++nb) hw |= (uint32_t)codes[c16 + 16 * nb] << (2 * nb);
  const int sl = info.slot_in_page;
  *reinterpret_cast<uint16_t*>(pages + info.rec + kVCodes + 8 * (16 * (sl / 4) + c16) +
                               4 * ((sl % 4) / 2) + 2 * (sl % 2)) = (uint16_t)hw;
}

// ------------------------------------------------------------------ exact fp64 (few rows)
//
// One workgroup = 16 consecutive new rows of one (KV head, K|V).  The 64 KiB rotation matrix is
// staged in LDS once per workgroup; each thread accumulates 2 rows x 4 output channels in fp64.

__global__ __launch_bounds__(kThreads) void rotate_quantize_append_kernel(
    CacheGeom g, uint8_t* __restrict__ pages, uint16_t* __restrict__ sinkwin,
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ slot_ids, int batch,
    int total_new, const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
    const int32_t* __restrict__ new_offsets, const int32_t* __restrict__ start_pos,
    const float* __restrict__ rot_k, const float* __restrict__ rot_v, float clip_k,
    float clip_v) {
#pragma clang fp contract(off)
  __shared__ float4 s_rot[kHeadDim * kHeadDim / 4];   // R[i][j], row-major, 64 KiB
  __shared__ float s_x[kRows][kHeadDim];              // input rows (bf16 widened)
  __shared__ float s_y[kRows][kHeadDim + 1];          // rotated rows (fp32)
  __shared__ uint8_t s_code[kRows][kHeadDim];
  __shared__ RowInfo s_info[kRows];

  const int t = threadIdx.x;
  const int row0 = blockIdx.x * kRows;
  const int h = blockIdx.y;
  const bool is_v = blockIdx.z != 0;
  const float* rot = (is_v ? rot_v : rot_k) + (size_t)h * kHeadDim * kHeadDim;
  const uint16_t* src = is_v ? v_new : k_new;
  const float clip = is_v ? clip_v : clip_k;
  const int nrows = min(kRows, total_new - row0);

  // Stage R (fp32) and the rows: all 16 loads of a thread are issued before the first LDS
  // store, so staging costs one memory latency.
  const float4* rot4 = reinterpret_cast<const float4*>(rot);
  {
    constexpr int kPer = kHeadDim * kHeadDim / 4 / kThreads;  // 16
    float4 rr[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) rr[k] = rot4[t + kThreads * k];
#pragma unroll
    for (int k = 0; k < kPer; ++k) s_rot[t + kThreads * k] = rr[k];
  }
  for (int i = t; i < kRows * kHeadDim; i += kThreads) {
    int r = i / kHeadDim, c = i % kHeadDim;
    s_x[r][c] = r < nrows ? bf16_to_f32(src[((size_t)(row0 + r) * g.hkv + h) * kHeadDim + c]) : 0.f;
  }
  if (t < kRows) {
    RowInfo info{-1, 0, -1};
    if (t < nrows)
      info = row_info(g, block_table, slot_ids, batch, new_offsets, start_pos, sinkwin != nullptr,
                      row0 + t, h, is_v);
    s_info[t] = info;
  }
  __syncthreads();

  // y = x . R: thread -> rows {2*rp, 2*rp+1}, channels 4*jq .. 4*jq+3; fp64, i ascending.
  {
    const int rp = t / 32, jq = t % 32;
    const int r0 = 2 * rp, r1 = 2 * rp + 1;
    double a0[4] = {0.0, 0.0, 0.0, 0.0}, a1[4] = {0.0, 0.0, 0.0, 0.0};
    for (int i = 0; i < kHeadDim; ++i) {
      const double x0 = (double)s_x[r0][i];
      const double x1 = (double)s_x[r1][i];
      const float4 rv = s_rot[i * (kHeadDim / 4) + jq];
      const double rr[4] = {(double)rv.x, (double)rv.y, (double)rv.z, (double)rv.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        a0[k] = __fma_rn(x0, rr[k], a0[k]);   // product exact in fp64: same as mul then add
        a1[k] = __fma_rn(x1, rr[k], a1[k]);
      }
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      s_y[r0][4 * jq + k] = (float)a0[k];
      s_y[r1][4 * jq + k] = (float)a1[k];
    }
  }
  __syncthreads();

  // Group parameters and codes: thread -> (row, group, quarter of the group's 32 channels).
  {
    const int r = t >> 4, gi = (t >> 2) & 3, sub = t & 3;
    const int c0 = gi * kGroup + 8 * sub;
    float mx = s_y[r][c0], mn = mx;
#pragma unroll
    for (int c = 1; c < 8; ++c) {
      const float v = s_y[r][c0 + c];
      mx = fmaxf(mx, v);
      mn = fminf(mn, v);
    }
    // the four quarters of the group are adjacent lanes
    mx = fmaxf(mx, __shfl_xor(mx, 1));
    mn = fminf(mn, __shfl_xor(mn, 1));
    mx = fmaxf(mx, __shfl_xor(mx, 2));
    mn = fminf(mn, __shfl_xor(mn, 2));
    _Float16 s16, z16;
    group_params(mx, mn, clip, s16, z16);
    const float sc = (float)s16, z = (float)z16;
#pragma unroll
    for (int c = 0; c < 8; ++c) s_code[r][c0 + c] = (uint8_t)code_of(s_y[r][c0 + c], sc, z);
    const RowInfo info = s_info[r];
    if (sub == 0 && r < nrows && info.rec >= 0) store_meta(pages, info, is_v, gi, meta_word(s16, z16));
  }
  __syncthreads();

  // Pack codes into the record.
  if (!is_v) {
    if (t < kRows * 8) {
      const int r = t / 8, d = t % 8;
      const RowInfo info = s_info[r];
      if (r < nrows && info.rec >= 0) store_k_word(pages, info, s_code[r], d);
    }
  } else {
    const int r = t / 16, c16 = t % 16;
    const RowInfo info = s_info[r];
    if (r < nrows && info.rec >= 0) store_v_half(pages, info, s_code[r], c16);
  }

  // BF16 sink/window rows.
  for (int i = t; i < kRows * kHeadDim; i += kThreads) {
    const int r = i / kHeadDim, c = i % kHeadDim;
    if (r < nrows && s_info[r].sw >= 0) sinkwin[s_info[r].sw + c] = f32_to_bf16_rne(s_y[r][c]);
  }
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
// 14.1 u ||x|| ||R_.j||.  The kernel uses E = 64 u ||x|| ||R_.j|| (the fp32 norms scaled up by
// 1.01 and 1.001) plus 2^-100 for flushed subnormals.
//
// Certification (each output is a monotone function of the values it reads):
//   * s16, z16 of a group: equal at the ends of the extremes' intervals [m - E, m + E], else
//     every channel that can be the extreme (within 2E of it) is recomputed as defined, after
//     which the extremes are the defined ones;
//   * a code: code_of equal at y - E and y + E, else y is recomputed;
//   * a BF16 copy (sink/window row): bf16 equal at y - E and y + E, else y is recomputed.
// Recomputed values are the defined ones (fp64, ascending, one rounding) and certify exactly,
// so every written byte equals the fp64 kernel's.
constexpr int kPTile = 64;
constexpr int kPThreads = 512;
constexpr int kXStride = kHeadDim + 8;   // bf16 per LDS row of x: 16-byte rows, skewed banks
constexpr int kYStride = kHeadDim + 4;   // floats per LDS row of y
constexpr int kExact = 0x80;             // s_code mark: s_y holds the defined value
constexpr float kErrUnits = 64.0f;
constexpr float kErrAbs = 0x1p-100f;

// The next fp32 value above / below a finite x (outward rounding of interval ends).
__device__ __forceinline__ float up(float x) {
  if (x == 0.0f) return __uint_as_float(1u);
  const uint32_t b = __float_as_uint(x);
  return __uint_as_float(x > 0.0f ? b + 1u : b - 1u);
}
__device__ __forceinline__ float down(float x) { return -up(-x); }

// The defined rotated value of (row r, channel c): fp64 sum over i ascending, rounded to fp32.
__device__ float defined_y(const uint16_t* xrow, const float* __restrict__ rot, int c) {
  double acc = 0.0;
  for (int i0 = 0; i0 < kHeadDim; i0 += 8) {
    const uint4 xv = *reinterpret_cast<const uint4*>(xrow + i0);
    float rv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) rv[e] = rot[(i0 + e) * kHeadDim + c];
    const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float xf = __uint_as_float(e & 1 ? xw[e / 2] & 0xFFFF0000u : xw[e / 2] << 16);
      acc = __fma_rn((double)xf, (double)rv[e], acc);
    }
  }
  return (float)acc;
}

__global__ __launch_bounds__(kPThreads, 4) void rotate_quantize_prefill_kernel(
    CacheGeom g, uint8_t* __restrict__ pages, uint16_t* __restrict__ sinkwin,
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ slot_ids, int batch,
    int total_new, const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
    const int32_t* __restrict__ new_offsets, const int32_t* __restrict__ start_pos,
    const float* __restrict__ rot_k, const float* __restrict__ rot_v, float clip_k,
    float clip_v) {
#pragma clang fp contract(off)
  __shared__ __attribute__((aligned(16))) uint16_t s_x[kPTile][kXStride];
  __shared__ __attribute__((aligned(16))) float s_y[kPTile][kYStride];
  __shared__ __attribute__((aligned(16))) uint8_t s_code[kPTile][kHeadDim];
  __shared__ RowInfo s_info[kPTile];
  __shared__ float s_err[kPTile];          // 64 u ||x|| (x 1.01) per row
  __shared__ float s_cn[kHeadDim];         // ||R_.j|| per output channel (rounded up)
  __shared__ float s_cng[kGroups];         // the largest of them per group
  __shared__ float2 s_sz[kPTile][kGroups]; // (scale, zero) as fp32
  __shared__ int s_n[2];                   // lengths of the two recompute lists
  __shared__ uint16_t s_list[kPTile * kHeadDim];  // (row, channel) to recompute: 128 r + c

  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int h = blockIdx.y;
  const bool is_v = blockIdx.z != 0;
  const float* rot = (is_v ? rot_v : rot_k) + (size_t)h * kHeadDim * kHeadDim;
  const uint16_t* src = is_v ? v_new : k_new;
  const float clip = is_v ? clip_v : clip_k;
  const int m = lane & 15, kq = lane >> 4;

  // A operands: lane (m, kq), slice s holds R[32s + 8kq + e][16w + m], e = 0..7, as 3 pieces.
  v8bf ra[4][3];
  {
    float ss = 0.f;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      float rv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) rv[e] = rot[(32 * s + 8 * kq + e) * kHeadDim + 16 * wave + m];
      uint16_t pc[3][8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float r0 = rv[e];
        ss = fmaf(r0, r0, ss);
        pc[0][e] = f32_to_bf16_rne(r0);
        const float r1 = r0 - bf16_to_f32(pc[0][e]);
        pc[1][e] = f32_to_bf16_rne(r1);
        const float r2 = r1 - bf16_to_f32(pc[1][e]);
        pc[2][e] = f32_to_bf16_rne(r2);
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
    ss += __shfl_xor(ss, 16);
    ss += __shfl_xor(ss, 32);
    if (kq == 0) s_cn[16 * wave + m] = __builtin_sqrtf(ss) * 1.001f;
  }
  __syncthreads();
  if (t < kGroups) {
    float cm = s_cn[kGroup * t];
    for (int c = 1; c < kGroup; ++c) cm = fmaxf(cm, s_cn[kGroup * t + c]);
    s_cng[t] = cm;
  }

  const int ntiles = (total_new + kPTile - 1) / kPTile;
  for (int tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
    const int row0 = tile * kPTile;
    const int nrows = min(kPTile, total_new - row0);

    // Input rows into LDS (8 threads per row, 2 x 16 bytes each), their norms, placements.
    {
      const int r = t >> 3, q = t & 7;
      uint4 u0 = {0, 0, 0, 0}, u1 = {0, 0, 0, 0};
      if (r < nrows) {
        const uint4* rp = reinterpret_cast<const uint4*>(src + ((size_t)(row0 + r) * g.hkv + h) * kHeadDim);
        u0 = rp[q];
        u1 = rp[q + 8];
      }
      *reinterpret_cast<uint4*>(&s_x[r][8 * q]) = u0;
      *reinterpret_cast<uint4*>(&s_x[r][8 * q + 64]) = u1;
      const uint32_t xw[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
      float ss = 0.f;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float a = __uint_as_float(xw[k] << 16), b = __uint_as_float(xw[k] & 0xFFFF0000u);
        ss = fmaf(a, a, ss);
        ss = fmaf(b, b, ss);
      }
      ss += __shfl_xor(ss, 1);
      ss += __shfl_xor(ss, 2);
      ss += __shfl_xor(ss, 4);
      if (q == 0) s_err[r] = kErrUnits * 0x1p-24f * 1.01f * __builtin_sqrtf(ss);
      if (t < kPTile) {
        RowInfo info{-1, 0, -1};
        if (t < nrows)
          info = row_info(g, block_table, slot_ids, batch, new_offsets, start_pos,
                          sinkwin != nullptr, row0 + t, h, is_v);
        s_info[t] = info;
      }
      if (t == 0) s_n[0] = s_n[1] = 0;
    }
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
      y.x = (acc[0][0] + acc[1][0]) + (acc[2][0] + acc[3][0]);
      y.y = (acc[0][1] + acc[1][1]) + (acc[2][1] + acc[3][1]);
      y.z = (acc[0][2] + acc[1][2]) + (acc[2][2] + acc[3][2]);
      y.w = (acc[0][3] + acc[1][3]) + (acc[2][3] + acc[3][3]);
      // D row = channel 16w + 4kq + i, column = token 16tt + m
      *reinterpret_cast<float4*>(&s_y[16 * tt + m][16 * wave + 4 * kq]) = y;
    }
    __syncthreads();

    // Thread -> (row r, group gi, half of the group's 32 channels) for the group passes.
    const int r = t >> 3, gi = (t >> 1) & 3, half = t & 1;
    const int c0 = gi * kGroup + 16 * half;
    const float er = s_err[r];

    // Pass 1: certify each group's scale and zero; if they are not certain, queue every channel
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
      const float cmax = s_cng[gi];
      const float E = up(er * cmax + kErrAbs);
      _Float16 s_hi, z_hi, s_lo, z_lo;
      group_params(up(mx + E), down(mn - E), clip, s_hi, z_lo);
      group_params(down(mx - E), up(mn + E), clip, s_lo, z_hi);
      const bool sure = __builtin_bit_cast(uint16_t, s_hi) == __builtin_bit_cast(uint16_t, s_lo) &&
                        __builtin_bit_cast(uint16_t, z_hi) == __builtin_bit_cast(uint16_t, z_lo);
      *reinterpret_cast<uint4*>(&s_code[r][c0]) = uint4{0, 0, 0, 0};
      if (!sure && r < nrows) {
        const float top = down(mx - 2.0f * E), bot = up(mn + 2.0f * E);
#pragma unroll
        for (int c = 0; c < 16; ++c)
          if (yv[c] >= top || yv[c] <= bot) s_list[atomicAdd(&s_n[0], 1)] = (uint16_t)(kHeadDim * r + c0 + c);
      }
    }
    __syncthreads();
    {
      const int n = s_n[0];
      for (int k = t; k < n; k += kPThreads) {
        const int it = s_list[k], rr = it / kHeadDim, c = it % kHeadDim;
        s_y[rr][c] = defined_y(&s_x[rr][0], rot, c);
        s_code[rr][c] = kExact;
      }
    }
    __syncthreads();

    // Pass 2: the group's scale and zero (now the defined ones), then every code and BF16 copy,
    // queueing the values the bound cannot certify.
    {
      float yv[16];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float4 a = *reinterpret_cast<const float4*>(&s_y[r][c0 + 4 * k]);
        yv[4 * k] = a.x; yv[4 * k + 1] = a.y; yv[4 * k + 2] = a.z; yv[4 * k + 3] = a.w;
      }
      const uint4 mk = *reinterpret_cast<const uint4*>(&s_code[r][c0]);
      const uint32_t mw[4] = {mk.x, mk.y, mk.z, mk.w};
      float mx = yv[0], mn = yv[0];
#pragma unroll
      for (int c = 1; c < 16; ++c) {
        mx = fmaxf(mx, yv[c]);
        mn = fminf(mn, yv[c]);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 1));
      mn = fminf(mn, __shfl_xor(mn, 1));
      _Float16 s16, z16;
      group_params(mx, mn, clip, s16, z16);
      const float sc = (float)s16, z = (float)z16;
      const RowInfo info = s_info[r];
      if (half == 0) {
        s_sz[r][gi] = make_float2(sc, z);
        if (r < nrows && info.rec >= 0) store_meta(pages, info, is_v, gi, meta_word(s16, z16));
      }
      const bool bf = info.sw >= 0;
      uint32_t cw[4] = {0, 0, 0, 0};
#pragma unroll
      for (int c = 0; c < 16; ++c) {
        const float y = yv[c];
        int code;
        bool ok = true;
        if (((mw[c / 4] >> (8 * (c % 4))) & 0xFF) == kExact) {
          code = code_of(y, sc, z);
        } else {
          const float E = up(er * s_cn[c0 + c] + kErrAbs);
          const float ylo = down(y - E), yhi = up(y + E);
          code = code_of(ylo, sc, z);
          ok = code == code_of(yhi, sc, z);
          if (bf) ok = ok && f32_to_bf16_rne(ylo) == f32_to_bf16_rne(yhi);
        }
        cw[c / 4] |= (uint32_t)code << (8 * (c % 4));
        if (!ok && r < nrows) s_list[atomicAdd(&s_n[1], 1)] = (uint16_t)(kHeadDim * r + c0 + c);
      }
      *reinterpret_cast<uint4*>(&s_code[r][c0]) = uint4{cw[0], cw[1], cw[2], cw[3]};
    }
    __syncthreads();
    {
      const int n = s_n[1];
      for (int k = t; k < n; k += kPThreads) {
        const int it = s_list[k], rr = it / kHeadDim, c = it % kHeadDim;
        const float y = defined_y(&s_x[rr][0], rot, c);
        const float2 sz = s_sz[rr][c / kGroup];
        s_y[rr][c] = y;
        s_code[rr][c] = (uint8_t)code_of(y, sz.x, sz.y);
      }
    }
    __syncthreads();

    // Pack the codes into the records; BF16 copies of sink/window rows.
    if (!is_v) {
      const int d = t & 7;
      const RowInfo info = s_info[r];
      if (r < nrows && info.rec >= 0) store_k_word(pages, info, s_code[r], d);
    } else {
      for (int e = t; e < kPTile * 16; e += kPThreads) {
        const int rr = e >> 4, c16 = e & 15;
        const RowInfo info = s_info[rr];
        if (rr < nrows && info.rec >= 0) store_v_half(pages, info, s_code[rr], c16);
      }
    }
    for (int e = t; e < kPTile * kHeadDim; e += kPThreads) {
      const int rr = e / kHeadDim, c = e % kHeadDim;
      if (rr < nrows && s_info[rr].sw >= 0) sinkwin[s_info[rr].sw + c] = f32_to_bf16_rne(s_y[rr][c]);
    }
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_append(const CacheGeom& g, uint8_t* pages, uint16_t* sinkwin,
                         const int32_t* block_table, const int32_t* slot_ids, int batch,
                         int total_new, const uint16_t* k_new, const uint16_t* v_new,
                         const int32_t* new_offsets, const int32_t* start_pos,
                         const float* rot_k, const float* rot_v, float clip_k, float clip_v,
                         int method, hipStream_t stream) {
  if (batch == 0 || total_new == 0) return hipSuccess;
  if (method == kAppendAuto) method = total_new >= kMatrixAppendRows ? kAppendMatrix : kAppendVector;
  if (method == kAppendMatrix) {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
      cus = 256;
    // two resident workgroups per CU over the 2 * Hkv (KV head, K|V) pairs
    const int tiles = (total_new + kPTile - 1) / kPTile;
    const int per_pair = max(1, min(tiles, (2 * cus + 2 * g.hkv - 1) / (2 * g.hkv)));
    hipLaunchKernelGGL(rotate_quantize_prefill_kernel, dim3(per_pair, g.hkv, 2), dim3(kPThreads), 0,
                       stream, g, pages, sinkwin, block_table, slot_ids, batch, total_new, k_new,
                       v_new, new_offsets, start_pos, rot_k, rot_v, clip_k, clip_v);
    return hipGetLastError();
  }
  dim3 grid((total_new + kRows - 1) / kRows, g.hkv, 2);
  hipLaunchKernelGGL(rotate_quantize_append_kernel, grid, dim3(kThreads), 0, stream, g, pages,
                     sinkwin, block_table, slot_ids, batch, total_new, k_new, v_new, new_offsets,
                     start_pos, rot_k, rot_v, clip_k, clip_v);
  return hipGetLastError();
}

}  // namespace oscar
