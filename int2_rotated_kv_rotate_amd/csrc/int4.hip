// INT4 variant of the cache: the same rotation, clipping, groups, sink/window store, workspace
// and combine, with 16-level codes in a 2560-byte record per (page, KV head).  The INT4 abstract
// on the OSCAR paper's page ("OSCAR: Offline Spectral Covariance-Aware Rotation for 2-bit KV
// Cache Quantization") finds token-wise INT4 with a rotation the serving-compatible choice at 4
// bits; this file carries that codec through the same paged path.
//
// Record (2560 bytes, 4-bit codes; the arrangement is this implementation's own, made for the
// matrix-core operands):
//   [   0, 1024)  K codes in 16-byte lane chunks: chunk 16 q + r holds slot r's channels
//                 16q .. 16q+15 (bytes 0..7) and 64+16q .. (bytes 8..15); channel c (h = c/64,
//                 q = (c%64)/16, j = c%16, i = j%4) at byte 16 (16q + r) + 8h + 4 (i/2) + j/4,
//                 bits 4 (i%2), so the 0x0F0F0F0F masks of a chunk give the INT2 record's int8
//                 operand order (byte b of vector i = channel 16q + 4b + i);
//   [1024, 2048)  V codes in 16-byte lane chunks: chunk 16 (r/4) + c%16, dword nb/2 (nb = c/16),
//                 byte 2 (u%2) + u/2 of it (u = r%4: each slot owns whole bytes), nibble nb%2;
//                 shifts of a dword by +3 / -5 (-1 / -9) masked with 0x00780078 give column
//                 block 2k's (2k+1's) codes of tokens 0,1 / 2,3 as bf16 1 + code/16 mantissas;
//   [2048, 2304)  K (fp16 scale, fp16 zero) of group g of slot r at 2048 + 16 r + 4 g;
//   [2304, 2560)  V (scale, zero), the same arrangement.
// Quantiser: s = fp16(fp32(c mx - c mn) / 15), z = fp16(c mn), code = clamp(rint((y - z) / s),
// 0, 15) in fp32 (0 when s == 0); y is the fp64 ascending rotation rounded once to fp32 (minus
// the optional key mean term, as in the INT2 append).
//
// Kernels:
//   int4_append_kernel  16 new rows of one (KV head, K|V) per workgroup, fp64 rotation on the
//                       vector ALUs (R staged in LDS), quantisation, packing, BF16 copies;
//                       appends of kMatrixAppendRows rows or more take the matrix-core prefill
//                       kernel of append.hip in its 4-bit form instead (the same bytes);
// The decode of these records runs on the matrix cores (int4_decode_mfma_kernel in decode.hip,
// every G), in the INT2 workspace format, so oscar_combine finishes it.
#include "oscar_internal.h"

namespace oscar {
namespace {

constexpr int kRecord4 = 2560;
constexpr int kK4Codes = 0, kV4Codes = 1024, kK4Meta = 2048, kV4Meta = 2304;
constexpr int kT4 = 256;

// grid (ceil(N / 16), Hkv, K|V), 256 threads.
__global__ __launch_bounds__(kT4) void int4_append_kernel(
    CacheGeom g, uint8_t* __restrict__ pages, uint16_t* __restrict__ sinkwin,
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ slot_ids, int batch,
    int total_new, const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
    const int32_t* __restrict__ new_offsets, const int32_t* __restrict__ start_pos,
    const float* __restrict__ rot_k, const float* __restrict__ rot_v,
    const float* __restrict__ k_mean, float clip_k, float clip_v) {
#pragma clang fp contract(off)
  constexpr int ROWS = 16;
  __shared__ float4 s_rot[kHeadDim * kHeadDim / 4];
  __shared__ float s_x[ROWS][kHeadDim];
  __shared__ float s_y[ROWS][kHeadDim + 1];
  __shared__ uint8_t s_code[ROWS][kHeadDim];
  __shared__ float s_mu[kHeadDim];
  __shared__ double s_c[kHeadDim];
  __shared__ RowInfo s_info[ROWS];

  const int t = threadIdx.x;
  const int row0 = blockIdx.x * ROWS;
  const int h = blockIdx.y;
  const bool is_v = blockIdx.z != 0;
  const float* rot = (is_v ? rot_v : rot_k) + (size_t)h * kHeadDim * kHeadDim;
  const uint16_t* src = is_v ? v_new : k_new;
  const float clip = is_v ? clip_v : clip_k;
  const int nrows = min(ROWS, total_new - row0);
  const bool centered = !is_v && k_mean != nullptr;

  {
    constexpr int kPer = kHeadDim * kHeadDim / 4 / kT4;
    const float4* rot4 = reinterpret_cast<const float4*>(rot);
    float4 rr[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) rr[k] = rot4[t + kT4 * k];
#pragma unroll
    for (int k = 0; k < kPer; ++k) s_rot[t + kT4 * k] = rr[k];
  }
  for (int i = t; i < ROWS * kHeadDim; i += kT4) {
    const int r = i / kHeadDim, c = i % kHeadDim;
    s_x[r][c] = r < nrows ? bf16_to_f32(src[((size_t)(row0 + r) * g.hkv + h) * kHeadDim + c]) : 0.f;
  }
  if (t < ROWS) {
    RowInfo info{-1, 0, -1};
    if (t < nrows)
      info = row_info_t<kRecord4>(g, block_table, slot_ids, batch, new_offsets, start_pos,
                                  sinkwin != nullptr, row0 + t, h, is_v);
    s_info[t] = info;
  }
  if (centered && t < kHeadDim) s_mu[t] = k_mean[(size_t)h * kHeadDim + t];
  __syncthreads();
  if (centered) {
    if (t < kHeadDim) {
      const float* rf = reinterpret_cast<const float*>(s_rot);
      double c = 0.0;
      for (int i = 0; i < kHeadDim; ++i) c = __fma_rn((double)s_mu[i], (double)rf[i * kHeadDim + t], c);
      s_c[t] = c;
    }
    __syncthreads();
  }

  // y = x . R, fp64, i ascending; thread -> rows 2rp, 2rp + 1, channels 4jq .. 4jq + 3
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
  }
  __syncthreads();

  // group parameters and codes: thread -> (row r, group gi, quarter sub: 8 channels)
  {
    const int r = t / 16, gi = (t / 4) % 4, sub = t % 4;
    const int c0 = gi * kGroup + 8 * sub;
    float mx = s_y[r][c0], mn = mx;
#pragma unroll
    for (int c = 1; c < 8; ++c) {
      const float v = s_y[r][c0 + c];
      mx = fmaxf(mx, v);
      mn = fminf(mn, v);
    }
#pragma unroll
    for (int o = 1; o < 4; o <<= 1) {
      mx = fmaxf(mx, __shfl_xor(mx, o));
      mn = fminf(mn, __shfl_xor(mn, o));
    }
    _Float16 s16, z16;
    group_params_t<15>(mx, mn, clip, s16, z16);
    const float sc = (float)s16, z = (float)z16;
#pragma unroll
    for (int c = 0; c < 8; ++c) s_code[r][c0 + c] = (uint8_t)code_of_t<15>(s_y[r][c0 + c], sc, z);
    const RowInfo info = s_info[r];
    if (sub == 0 && r < nrows && info.rec >= 0)
      *reinterpret_cast<uint32_t*>(pages + info.rec + (is_v ? kV4Meta : kK4Meta) +
                                   16 * info.slot_in_page + 4 * gi) =
          (uint32_t)__builtin_bit_cast(uint16_t, s16) |
          ((uint32_t)__builtin_bit_cast(uint16_t, z16) << 16);
  }
  __syncthreads();

  // packing (thread -> row t / 16, w = t % 16), BF16 copies.  K: w = 4 q + d is dword d of the
  // row's chunk q, byte b = channels 64 (d/2) + 16 q + 4 b + 2 (d%2) and + 1 (low, high nibble).
  // V: w is the channel residue; the row owns byte 2 (u%2) + u/2 of each dword k of chunk
  // 16 (slot/4) + w, the codes of channels 32 k + w (low nibble) and 32 k + 16 + w (high).
  {
    const int r = t / 16, w = t % 16;
    const RowInfo info = s_info[r];
    if (r < nrows && info.rec >= 0) {
      const int sl = info.slot_in_page;
      if (!is_v) {
        const int q = w >> 2, d = w & 3;
        const int cb = 64 * (d >> 1) + 16 * q + 2 * (d & 1);
        uint32_t word = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b)
          word |= ((uint32_t)s_code[r][cb + 4 * b] | ((uint32_t)s_code[r][cb + 4 * b + 1] << 4))
                  << (8 * b);
        *reinterpret_cast<uint32_t*>(pages + info.rec + kK4Codes + 16 * (16 * q + sl) + 4 * d) = word;
      } else {
        const int u = sl & 3;
        uint8_t* chunk = pages + info.rec + kV4Codes + 16 * (16 * (sl >> 2) + w) + 2 * (u & 1) + (u >> 1);
#pragma unroll
        for (int k = 0; k < 4; ++k)
          chunk[4 * k] = (uint8_t)(s_code[r][32 * k + w] | (s_code[r][32 * k + 16 + w] << 4));
      }
    }
    if (r < nrows && info.sw >= 0) {
      const float* yr = &s_y[r][8 * w];
      uint32_t o[4];
#pragma unroll
      for (int k = 0; k < 4; ++k)
        o[k] = f32_to_bf16_rne(yr[2 * k]) | ((uint32_t)f32_to_bf16_rne(yr[2 * k + 1]) << 16);
      *reinterpret_cast<uint4*>(sinkwin + info.sw + 8 * w) = uint4{o[0], o[1], o[2], o[3]};
    }
  }
}

}  // namespace

hipError_t launch_int4_append(const CacheGeom& g, uint8_t* pages, uint16_t* sinkwin,
                              const int32_t* block_table, const int32_t* slot_ids, int batch,
                              int total_new, const uint16_t* k_new, const uint16_t* v_new,
                              const int32_t* new_offsets, const int32_t* start_pos,
                              const float* rot_k, const float* rot_v, const float* k_mean,
                              float clip_k, float clip_v, hipStream_t stream) {
  if (batch == 0 || total_new == 0) return hipSuccess;
  // prefill-sized appends on the matrix cores (certified, the same bytes: append.hip)
  if (total_new >= kMatrixAppendRows)
    return launch_prefill_int4(g, pages, sinkwin, block_table, slot_ids, batch, total_new, k_new,
                               v_new, new_offsets, start_pos, rot_k, rot_v, k_mean, clip_k, clip_v,
                               stream);
  hipLaunchKernelGGL(int4_append_kernel, dim3((total_new + 15) / 16, g.hkv, 2), dim3(kT4), 0,
                     stream, g, pages, sinkwin, block_table, slot_ids, batch, total_new, k_new,
                     v_new, new_offsets, start_pos, rot_k, rot_v, k_mean, clip_k, clip_v);
  return hipGetLastError();
}

hipError_t launch_int4_decode(const CacheGeom& g, const uint8_t* pages, const uint16_t* sinkwin,
                              const int32_t* block_table, const int32_t* slot_ids, int batch,
                              int hq, const uint16_t* q, const int32_t* seq_lens,
                              const float* rot_k, float sm_scale, int split_pages,
                              const Workspace& ws, hipStream_t stream) {
  (void)split_pages;   // the matrix-core kernel's stream-K workers need no split size
  if (batch == 0) return hipSuccess;
  return launch_int4_mfma_decode(g, pages, sinkwin, block_table, slot_ids, batch, hq, q, seq_lens,
                                 rot_k, sm_scale, ws, stream);
}

}  // namespace oscar
