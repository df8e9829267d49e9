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
//   int4_decode_kernel  (G = 8; G <= 4 runs int4_decode_mfma_kernel on the matrix cores, in
//                       decode.hip) one workgroup per (split, KV head, sequence): every position of the
//                       split, INT4 or BF16 sink/window, on the vector ALUs; each of the 16
//                       token lanes keeps its own running softmax (rescaled only when its max
//                       grows) and the 16 are merged at the end; the next page's words are
//                       loaded while a page is computed; writes a partial in the INT2 workspace
//                       format, so oscar_combine finishes it (R_V^T, fixed merge order).
#include "oscar_internal.h"

namespace oscar {
namespace {

constexpr int kRecord4 = 2560;
constexpr int kK4Codes = 0, kV4Codes = 1024, kK4Meta = 2048, kV4Meta = 2304;
constexpr int kT4 = 256;
constexpr float kLog2e4 = 1.4426950408889634f;
constexpr float kNegBig4 = -1.0e30f;

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

// ------------------------------------------------------------------------------------ decode

// grid (max_splits, Hkv, B), 256 threads: thread t = (token lane r = t / 16, channel octet
// k = t % 16: channels 8k .. 8k + 7, group k / 4).  Split s of sequence b covers pages
// [s * sp, (s + 1) * sp) with sp = max(split_pages, ceil(P_b / max_splits)), P_b = ceil(L_b / 16).
template <int GMAX>
__global__ __launch_bounds__(kT4, GMAX <= 4 ? 4 : 2) void int4_decode_kernel(
    CacheGeom g, const uint8_t* __restrict__ pages, const uint16_t* __restrict__ sinkwin,
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ slot_ids, int hq,
    const int32_t* __restrict__ seq_lens, float sm_scale, int split_pages, Workspace ws) {
  const int s = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int r = t >> 4, k = t & 15, gi = k >> 2;
  const int G = hq / g.hkv;
  const int max_splits = ws.max_splits();
  const int L = max(seq_lens[b], 0);
  const int P = (L + kPage - 1) / kPage;
  const int sp = max(split_pages, (P + max_splits - 1) / max_splits);
  const int nsplit = P == 0 ? 0 : (P + sp - 1) / sp;
  if (s == 0) {  // the split count of this pair, and empty window slots (positions are here)
    if (t == 0) ws.nvalid()[b * g.hkv + h] = nsplit;
    static_assert(GMAX * kWinSlots <= kT4, "one thread per empty window slot");
    if (t < G * kWinSlots)
      *ws.ml(b, hq, h * G + t / kWinSlots, ws.win_slot() + t % kWinSlots) = make_float2(kNegBig4, 0.f);
  }
  if (s >= nsplit) return;

  __shared__ float s_q[GMAX][kHeadDim];
  __shared__ float s_m[16][GMAX];
  __shared__ float s_acc[4][GMAX][kHeadDim];
  __shared__ float s_l[4][GMAX];
  for (int i = t; i < G * kHeadDim; i += kT4) {
    const float* qrow = reinterpret_cast<const float*>(ws.qblock(b, hq, h * G + i / kHeadDim));
    s_q[i / kHeadDim][i % kHeadDim] = qrow[i % kHeadDim];
  }
  __syncthreads();
  float qv[GMAX][8];
#pragma unroll
  for (int j = 0; j < GMAX; ++j)
#pragma unroll
    for (int c = 0; c < 8; ++c) qv[j][c] = j < G ? s_q[j][8 * k + c] : 0.f;

  const float sm_log2 = sm_scale * kLog2e4;
  const int n_sink = min(L, g.num_sink);
  const int n_win = min(g.window, L - n_sink);
  const int slot = slot_ids ? slot_ids[b] : b;
  const bool have_store = sinkwin != nullptr && slot >= 0 && slot < g.num_slots;
  const size_t sw_base = ((size_t)slot * g.hkv + h) * (size_t)(g.num_sink + g.window);
  float m[GMAX], l[GMAX], acc[GMAX][8];
#pragma unroll
  for (int j = 0; j < GMAX; ++j) {
    m[j] = kNegBig4;
    l[j] = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[j][c] = 0.f;
  }
  const int pg0 = s * sp, pg1 = min(P, pg0 + sp);
  // One position's words: kind 0 none, 1 BF16 store row (K, V octets), 2 INT4 record (codes and
  // (scale, zero) words).  Fetched one page ahead of its use.
  struct Words {
    int kind;
    uint4 ku, vu;
    uint32_t km, vm;
  };
  const int32_t* bt = block_table + (size_t)b * g.max_pages;
  auto fetch = [&](int pg) {
    Words f{0, make_uint4(0u, 0u, 0u, 0u), make_uint4(0u, 0u, 0u, 0u), 0u, 0u};
    const int pos = pg * kPage + r;
    if (pg >= pg1 || pos >= L) return f;
    if (pos < n_sink || pos >= L - n_win) {
      if (!have_store) return f;
      const int row = pos < n_sink ? pos : g.num_sink + pos % g.window;
      const uint16_t* kr = sinkwin + (sw_base + row) * 2 * kHeadDim;
      f.ku = *reinterpret_cast<const uint4*>(kr + 8 * k);
      f.vu = *reinterpret_cast<const uint4*>(kr + kHeadDim + 8 * k);
      f.kind = 1;
      return f;
    }
    const int id = pg < g.max_pages ? bt[pg] : -1;
    if (id < 0 || id >= g.num_pages) return f;
    const uint8_t* rec = pages + ((size_t)id * g.hkv + h) * kRecord4;
    // this lane's 8 channels 8k .. 8k+7 of slot r as one word, channel 8k + m at bits 4m.
    // K: bytes 2 (k%2) and 2 (k%2) + 1 of the two dwords of chunk 16 ((k%8)/2) + r, half k/8
    // (channels m = 0, 1, 4, 5 in the first dword, 2, 3, 6, 7 in the second).
    {
      const uint2 d = *reinterpret_cast<const uint2*>(rec + kK4Codes + 16 * (16 * ((k & 7) >> 1) + r) +
                                                      8 * (k >> 3));
      const uint32_t x = (d.x >> (16 * (k & 1))) & 0xFFFFu, y = (d.y >> (16 * (k & 1))) & 0xFFFFu;
      f.ku.x = (x & 0xFFu) | ((y & 0xFFu) << 8) | ((x >> 8) << 16) | ((y >> 8) << 24);
    }
    // V: channel 8k + m is residue 8 (k%2) + m of column block k/2: one byte per channel.
    {
      const int u = r & 3, e = (k >> 1) & 1;
      const uint8_t* vb = rec + kV4Codes + 16 * (16 * (r >> 2) + 8 * (k & 1)) + 4 * (k >> 2) +
                          2 * (u & 1) + (u >> 1);
      uint32_t word = 0;
#pragma unroll
      for (int m = 0; m < 8; ++m) word |= (((uint32_t)vb[16 * m] >> (4 * e)) & 15u) << (4 * m);
      f.vu.x = word;
    }
    f.km = *reinterpret_cast<const uint32_t*>(rec + kK4Meta + 16 * r + 4 * gi);
    f.vm = *reinterpret_cast<const uint32_t*>(rec + kV4Meta + 16 * r + 4 * gi);
    f.kind = 2;
    return f;
  };
  Words cur = fetch(pg0);
  for (int pg = pg0; pg < pg1; ++pg) {
    const Words nxt = fetch(pg + 1);
    if (cur.kind != 0) {   // the 16 lanes of a token agree
      float kx[8], vx[8];
      if (cur.kind == 1) {
        const uint32_t kw[4] = {cur.ku.x, cur.ku.y, cur.ku.z, cur.ku.w};
        const uint32_t vw[4] = {cur.vu.x, cur.vu.y, cur.vu.z, cur.vu.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          kx[2 * i] = __uint_as_float(kw[i] << 16);
          kx[2 * i + 1] = __uint_as_float(kw[i] & 0xFFFF0000u);
          vx[2 * i] = __uint_as_float(vw[i] << 16);
          vx[2 * i + 1] = __uint_as_float(vw[i] & 0xFFFF0000u);
        }
      } else {
        const float ks = (float)__builtin_bit_cast(_Float16, (uint16_t)(cur.km & 0xFFFFu));
        const float kz = (float)__builtin_bit_cast(_Float16, (uint16_t)(cur.km >> 16));
        const float vs = (float)__builtin_bit_cast(_Float16, (uint16_t)(cur.vm & 0xFFFFu));
        const float vz = (float)__builtin_bit_cast(_Float16, (uint16_t)(cur.vm >> 16));
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          kx[c] = fmaf(ks, (float)((cur.ku.x >> (4 * c)) & 15u), kz);
          vx[c] = fmaf(vs, (float)((cur.vu.x >> (4 * c)) & 15u), vz);
        }
      }
#pragma unroll
      for (int j = 0; j < GMAX; ++j) {
        if (j >= G) break;
        float d = 0.f;
#pragma unroll
        for (int c = 0; c < 8; ++c) d = fmaf(qv[j][c], kx[c], d);
        d += lane_xor_f32<1>(d);
        d += lane_xor_f32<2>(d);
        d += lane_xor_f32<4>(d);
        d += lane_xor_f32<8>(d);
        const float z = d * sm_log2;
        if (z > m[j]) {   // a new running max for this token lane: rescale its sums
          const float sc = __builtin_amdgcn_exp2f(m[j] - z);
          l[j] *= sc;
#pragma unroll
          for (int c = 0; c < 8; ++c) acc[j][c] *= sc;
          m[j] = z;
        }
        const float p = __builtin_amdgcn_exp2f(z - m[j]);
        l[j] += p;
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[j][c] = fmaf(p, vx[c], acc[j][c]);
      }
    }
    cur = nxt;
  }

  // merge the 16 token lanes: max of m over r, rescale, sum over the lanes of a wave (4 token
  // lanes), then over the 4 waves, in a fixed order
  if (k == 0) {
#pragma unroll
    for (int j = 0; j < GMAX; ++j)
      if (j < G) s_m[r][j] = m[j];
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < GMAX; ++j) {
    if (j >= G) break;
    float M = s_m[0][j];
    for (int rr = 1; rr < 16; ++rr) M = fmaxf(M, s_m[rr][j]);
    const float e = l[j] > 0.f ? __builtin_amdgcn_exp2f(m[j] - M) : 0.f;
    float lj = l[j] * e;
    lj += __shfl_xor(lj, 16);
    lj += __shfl_xor(lj, 32);
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      float a = acc[j][c] * e;
      a += __shfl_xor(a, 16);
      a += __shfl_xor(a, 32);
      acc[j][c] = a;
    }
    if (lane < 16) {
#pragma unroll
      for (int c = 0; c < 8; ++c) s_acc[wave][j][8 * k + c] = acc[j][c];
      if (k == 0) s_l[wave][j] = lj;
    }
    m[j] = M;
  }
  __syncthreads();
  for (int e = t; e < G * kHeadDim; e += kT4) {
    const int j = e / kHeadDim, c = e % kHeadDim;
    const float o = ((s_acc[0][j][c] + s_acc[1][j][c]) + s_acc[2][j][c]) + s_acc[3][j][c];
    const float lsum = ((s_l[0][j] + s_l[1][j]) + s_l[2][j]) + s_l[3][j];
    ws.o(b, hq, h * G + j, s)[c] = lsum > 0.f ? o : 0.f;
    if (c == 0) {
      float M = s_m[0][j];
      for (int rr = 1; rr < 16; ++rr) M = fmaxf(M, s_m[rr][j]);
      *ws.ml(b, hq, h * G + j, s) = make_float2(M, lsum);
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
  if (batch == 0) return hipSuccess;
  if (hq / g.hkv <= 4)   // the matrix-core kernel (stream-K workers; split_pages unused)
    return launch_int4_mfma_decode(g, pages, sinkwin, block_table, slot_ids, batch, hq, q,
                                   seq_lens, rot_k, sm_scale, ws, stream);
  hipError_t e = launch_prep_q(g, q, rot_k, batch, hq, seq_lens, ws, stream);
  if (e != hipSuccess) return e;
  const dim3 grid(ws.max_splits(), g.hkv, batch);
  if (hq / g.hkv <= 4)
    hipLaunchKernelGGL(int4_decode_kernel<4>, grid, dim3(kT4), 0, stream, g, pages, sinkwin,
                       block_table, slot_ids, hq, seq_lens, sm_scale, split_pages, ws);
  else
    hipLaunchKernelGGL(int4_decode_kernel<8>, grid, dim3(kT4), 0, stream, g, pages, sinkwin,
                       block_table, slot_ids, hq, seq_lens, sm_scale, split_pages, ws);
  return hipGetLastError();
}

}  // namespace oscar
