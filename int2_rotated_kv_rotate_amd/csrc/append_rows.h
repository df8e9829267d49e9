// The INT2 record helpers and the exact (fp64, vector-ALU) rotate-clip-quantize-append of a
// few rows, shared by the append kernels (append.hip) and the decode-step launch that runs the
// append beside the query preparation (step.hip).  Both translation units are built without
// floating-point contraction; the function also states it, because the quantiser is an fp32
// formula reproduced bit for bit.
//
// Method: OSCAR project card "FutureMLS-Lab/OSCAR", section "How it works" (fixed per-layer
// rotations and clipping thresholds, INT2 bulk, BF16 sink and recent window); OSCAR paper,
// "Abstract" (rotation + clipping computed offline and applied as fixed parameters).
#pragma once
#include "oscar_internal.h"

namespace oscar {
namespace {

// The INT2 forms of the shared helpers: 1536-byte records, 4 levels.
__device__ __forceinline__ RowInfo row_info(const CacheGeom& g, const int32_t* __restrict__ block_table,
                                            const int32_t* __restrict__ slot_ids, int batch,
                                            const int32_t* __restrict__ new_offsets,
                                            const int32_t* __restrict__ start_pos, bool has_store,
                                            int n, int h, bool is_v) {
  return row_info_t<kRecord>(g, block_table, slot_ids, batch, new_offsets, start_pos, has_store, n,
                             h, is_v);
}
__device__ __forceinline__ void group_params(float mx, float mn, float clip, _Float16& s16,
                                             _Float16& z16) {
  group_params_t<3>(mx, mn, clip, s16, z16);
}
__device__ __forceinline__ int code_of(float y, float s, float z) { return code_of_t<3>(y, s, z); }

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
// One workgroup = ROWS consecutive new rows of one (KV head, K|V).  The 64 KiB rotation matrix
// is staged in LDS once per workgroup.  ROWS = 16: each thread accumulates 2 rows x 4 output
// channels in fp64; ROWS = 4 (small appends, e.g. one decoded token per sequence, so that the
// launch spreads over more CUs): each thread accumulates 1 row x 2 channels.

constexpr int kAppendThreads = 256;

// Shared memory of one workgroup of append_rows.
template <int ROWS>
struct AppendShared {
  float4 rot[kHeadDim * kHeadDim / 4];  // R[i][j], row-major, 64 KiB
  float x[ROWS][kHeadDim];              // input rows (bf16 widened)
  float mu[kHeadDim];                   // key mean (centered K only)
  double c[kHeadDim];                   // C = mu . R, fp64
  float y[ROWS][kHeadDim + 1];          // rotated rows (fp32)
  uint8_t code[ROWS][kHeadDim];
  RowInfo info[ROWS];
};

// Workgroup (bx, by, bz) of the append: rows bx*ROWS .. of KV head by, K (bz = 0) or V (bz = 1);
// kAppendThreads threads.
template <int ROWS>
__device__ __forceinline__ void append_rows(
    const CacheGeom& g, uint8_t* __restrict__ pages, uint16_t* __restrict__ sinkwin,
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ slot_ids, int batch,
    int total_new, const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
    const int32_t* __restrict__ new_offsets, const int32_t* __restrict__ start_pos,
    const float* __restrict__ rot_k, const float* __restrict__ rot_v,
    const float* __restrict__ k_mean, float clip_k, float clip_v, int bx, int by, int bz,
    AppendShared<ROWS>& sm) {
#pragma clang fp contract(off)
  static_assert(ROWS == 4 || ROWS == 16, "row blocking");
  float4* s_rot = sm.rot;
  float (&s_x)[ROWS][kHeadDim] = sm.x;
  float* s_mu = sm.mu;
  double* s_c = sm.c;
  float (&s_y)[ROWS][kHeadDim + 1] = sm.y;
  uint8_t (&s_code)[ROWS][kHeadDim] = sm.code;
  RowInfo* s_info = sm.info;

  const int t = threadIdx.x;
  const int row0 = bx * ROWS;
  const int h = by;
  const bool is_v = bz != 0;
  const float* rot = (is_v ? rot_v : rot_k) + (size_t)h * kHeadDim * kHeadDim;
  const uint16_t* src = is_v ? v_new : k_new;
  const float clip = is_v ? clip_v : clip_k;
  const int nrows = min(ROWS, total_new - row0);
  const bool centered = !is_v && k_mean != nullptr;

  // Stage R (fp32) and the rows: the first round of the row placement lookups, all 16 R loads
  // of a thread and its input values are issued before the first wait, so staging costs about
  // two memory latencies (the lookups' second round overlaps the R loads).
  const bool look = t < nrows;  // t < ROWS
  RowLookup lk{};
  if (look) lk = row_lookup(new_offsets, start_pos, slot_ids, batch, row0 + t);
  const float4* rot4 = reinterpret_cast<const float4*>(rot);
  constexpr int kPer = kHeadDim * kHeadDim / 4 / kAppendThreads;  // 16
  float4 rr[kPer];
#pragma unroll
  for (int k = 0; k < kPer; ++k) rr[k] = rot4[t + kAppendThreads * k];
  constexpr int kXPer = ROWS * kHeadDim / kAppendThreads;  // 2 or 8
  uint16_t xv[kXPer];
#pragma unroll
  for (int k = 0; k < kXPer; ++k) {
    const int i = t + kAppendThreads * k, r = i / kHeadDim, c = i % kHeadDim;
    xv[k] = r < nrows ? src[((size_t)(row0 + r) * g.hkv + h) * kHeadDim + c] : (uint16_t)0;
  }
  if (t < ROWS) {
    RowInfo info{-1, 0, -1};
    if (look)
      info = row_info_from<kRecord>(g, block_table, slot_ids, batch, new_offsets, start_pos,
                                    sinkwin != nullptr, lk, h, is_v);
    s_info[t] = info;
  }
#pragma unroll
  for (int k = 0; k < kPer; ++k) s_rot[t + kAppendThreads * k] = rr[k];
#pragma unroll
  for (int k = 0; k < kXPer; ++k) {
    const int i = t + kAppendThreads * k;
    s_x[i / kHeadDim][i % kHeadDim] = bf16_to_f32(xv[k]);
  }
  if (centered && t < kHeadDim) s_mu[t] = k_mean[(size_t)h * kHeadDim + t];
  __syncthreads();
  // Key mean: C_j = sum_i mu_i R_ij in fp64, i ascending (exact products), removed from the
  // rotated key as one fp64 subtraction before the rounding to fp32.
  if (centered) {
    if (t < kHeadDim) {
      const float* rf = reinterpret_cast<const float*>(s_rot);
      double c = 0.0;
      for (int i = 0; i < kHeadDim; ++i) c = __fma_rn((double)s_mu[i], (double)rf[i * kHeadDim + t], c);
      s_c[t] = c;
    }
    __syncthreads();
  }

  // y = x . R in fp64, i ascending (products are exact in fp64: fma == mul then add).
  if constexpr (ROWS == 16) {
    // thread -> rows {2*rp, 2*rp+1}, channels 4*jq .. 4*jq+3
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
        a0[k] = __fma_rn(x0, rr[k], a0[k]);
        a1[k] = __fma_rn(x1, rr[k], a1[k]);
      }
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const double c = centered ? s_c[4 * jq + k] : 0.0;
      s_y[r0][4 * jq + k] = (float)(a0[k] - c);
      s_y[r1][4 * jq + k] = (float)(a1[k] - c);
    }
  } else {
    // thread -> row t / 64, channels 2*jp, 2*jp + 1
    const int rr = t / 64, jp = t % 64;
    const float2* rot2 = reinterpret_cast<const float2*>(s_rot);
    double a[2] = {0.0, 0.0};
#pragma unroll 8
    for (int i = 0; i < kHeadDim; ++i) {
      const double x = (double)s_x[rr][i];
      const float2 rv = rot2[i * (kHeadDim / 2) + jp];
      a[0] = __fma_rn(x, (double)rv.x, a[0]);
      a[1] = __fma_rn(x, (double)rv.y, a[1]);
    }
    const double c0 = centered ? s_c[2 * jp] : 0.0, c1 = centered ? s_c[2 * jp + 1] : 0.0;
    s_y[rr][2 * jp] = (float)(a[0] - c0);
    s_y[rr][2 * jp + 1] = (float)(a[1] - c1);
  }
  __syncthreads();

  // Group parameters and codes: SUB threads per (row, group), adjacent lanes.
  {
    constexpr int kSub = kAppendThreads / (ROWS * kGroups);   // 4 (ROWS = 16) or 16 (ROWS = 4)
    constexpr int kPerSub = kGroup / kSub;               // 8 or 2 channels each
    const int r = t / (kSub * kGroups), gi = (t / kSub) % kGroups, sub = t % kSub;
    const int c0 = gi * kGroup + kPerSub * sub;
    float mx = s_y[r][c0], mn = mx;
#pragma unroll
    for (int c = 1; c < kPerSub; ++c) {
      const float v = s_y[r][c0 + c];
      mx = fmaxf(mx, v);
      mn = fminf(mn, v);
    }
#pragma unroll
    for (int o = 1; o < kSub; o <<= 1) {
      mx = fmaxf(mx, __shfl_xor(mx, o));
      mn = fminf(mn, __shfl_xor(mn, o));
    }
    _Float16 s16, z16;
    group_params(mx, mn, clip, s16, z16);
    const float sc = (float)s16, z = (float)z16;
#pragma unroll
    for (int c = 0; c < kPerSub; ++c) s_code[r][c0 + c] = (uint8_t)code_of(s_y[r][c0 + c], sc, z);
    const RowInfo info = s_info[r];
    if (sub == 0 && r < nrows && info.rec >= 0) store_meta(pages, info, is_v, gi, meta_word(s16, z16));
  }
  __syncthreads();

  // Pack codes into the record.
  if (!is_v) {
    if (t < ROWS * 8) {
      const int r = t / 8, d = t % 8;
      const RowInfo info = s_info[r];
      if (r < nrows && info.rec >= 0) store_k_word(pages, info, s_code[r], d);
    }
  } else if (t < ROWS * 16) {
    const int r = t / 16, c16 = t % 16;
    const RowInfo info = s_info[r];
    if (r < nrows && info.rec >= 0) store_v_half(pages, info, s_code[r], c16);
  }

  // BF16 sink/window rows.
  for (int i = t; i < ROWS * kHeadDim; i += kAppendThreads) {
    const int r = i / kHeadDim, c = i % kHeadDim;
    if (r < nrows && s_info[r].sw >= 0) sinkwin[s_info[r].sw + c] = f32_to_bf16_rne(s_y[r][c]);
  }
}

}  // namespace
}  // namespace oscar
