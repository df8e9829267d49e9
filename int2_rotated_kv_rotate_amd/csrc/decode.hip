// Mixed-precision paged decode attention over the rotated INT2 cache.
//
// Method: OSCAR project card "FutureMLS-Lab/OSCAR", section "How it works" (BF16 sinks + BF16
// recent window + INT2 bulk, fused mixed-precision flash attention); OSCAR paper, "Abstract"
// (INT2 attention kernel that keeps the paged KV-cache layout; speed comes from reading fewer
// bytes).  Attention is computed in the rotated frame: q' = q . R_K makes q'.k' = q.k for
// orthogonal R_K, and the rotated output is rotated back with R_V^T by the combine kernel.
//
// Kernels
//   q_prep_kernel      per (sequence, KV head): q' = q . R_K for the G query heads of the group,
//                      plus an exact-integer form of q' for the int8 matrix cores.
//   int2_decode_kernel per (split, KV head, sequence), one wavefront: walks the split's pages
//                      through the block table.  Per page it reads one 1536-byte record with
//                      four coalesced vector loads per lane, computes the G x 16 logits on the
//                      int8 MFMA (codes are exact int8, q' is two int8 pieces), runs the online
//                      softmax, and accumulates P.V on the bf16 MFMA (codes exact as bf16
//                      1 + code/4, weights p*scale as two bf16 pieces).  The last split index
//                      handles the BF16 sink + window positions with fp32 VALU math.
//
// MFMA operand layouts (16x16 tiles, wave64): an A operand row m lives in lane m + 16*k4 and a
// B operand column n in lane n + 16*k4, with k4 selecting a quarter of the K dimension; the
// 16x16 result puts rows 4*(lane/16) + i of column lane%16 in accumulator register i.  The K
// axis is permuted consistently on both operands, which leaves the product unchanged.
#include "oscar_internal.h"

namespace oscar {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef short v4s __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegBig = -1.0e30f;

// ------------------------------------------------------------------------------- q prep

// grid (Hkv, batch), block 128 (thread = output channel).
__global__ __launch_bounds__(128) void q_prep_kernel(const uint16_t* __restrict__ q,
                                                    const float* __restrict__ rot_k, int hq,
                                                    int hkv, Workspace ws) {
  const int h = blockIdx.x, b = blockIdx.y, c = threadIdx.x;
  const int G = hq / hkv;
  __shared__ float s_q[8][kHeadDim];
  __shared__ float s_red[8][4];
  for (int j = 0; j < G; ++j)
    s_q[j][c] = bf16_to_f32(q[((size_t)b * hq + h * G + j) * kHeadDim + c]);
  __syncthreads();
  const float* R = rot_k + (size_t)h * kHeadDim * kHeadDim;
  float acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0.f;
  for (int i = 0; i < kHeadDim; ++i) {
    const float r = R[i * kHeadDim + c];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (j < G) acc[j] = fmaf(s_q[j][i], r, acc[j]);
  }
  // per-head max |q'| (over both waves) and per-group sums (group = 32-lane half of a wave)
  __shared__ float s_amax[8][2];
  const int lane = c & 63, wv = c >> 6;
  for (int j = 0; j < G; ++j) {
    float a = fabsf(acc[j]);
    float s = acc[j];
    for (int o = 16; o >= 1; o >>= 1) s += __shfl_xor(s, o);
    for (int o = 32; o >= 1; o >>= 1) a = fmaxf(a, __shfl_xor(a, o));
    if (lane == 0) s_red[j][2 * wv + 0] = s;
    if (lane == 32) s_red[j][2 * wv + 1] = s;
    if (lane == 0) s_amax[j][wv] = a;
  }
  __syncthreads();
  for (int j = 0; j < G; ++j) {
    const float amax = fmaxf(s_amax[j][0], s_amax[j][1]);
    const float qsc = amax / 127.0f;
    char* blk = ws.qblock(b, hq, h * G + j);
    const float v = acc[j];
    int hi = 0, lo = 0;
    if (qsc > 0.f) {
      hi = (int)__builtin_rintf(v / qsc);
      hi = max(-127, min(127, hi));
      const float r = v - (float)hi * qsc;
      lo = (int)__builtin_rintf(r * 254.0f / qsc);
      lo = max(-127, min(127, lo));
    }
    // slot order inside each 16-channel word: slot 4*i + b holds channel 4*b + i
    const int pos = 16 * (c / 16) + 4 * (c % 4) + (c % 16) / 4;
    reinterpret_cast<float*>(blk)[c] = v;
    blk[kQHiOff + pos] = (char)hi;
    blk[kQLoOff + pos] = (char)lo;
    if (c == 0) {
      *reinterpret_cast<float*>(blk + kQScOff) = qsc;
      float* qs = reinterpret_cast<float*>(blk + kQSumOff);
      qs[0] = s_red[j][0];
      qs[1] = s_red[j][1];
      qs[2] = s_red[j][2];
      qs[3] = s_red[j][3];
    }
  }
}

// ---------------------------------------------------------------------- small wave helpers

__device__ __forceinline__ float dpp_quad_xor1(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ float dpp_quad_xor2(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, false));
}
__device__ __forceinline__ float max_across_rows(float x) {  // lanes l, l^16, l^32, l^48
  x = fmaxf(x, __shfl_xor(x, 16));
  x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}
__device__ __forceinline__ float sum_across_rows(float x) {
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}

// bf16 "1 + code/4" for two 2-bit codes at bits (2*nb) and (16 + 2*nb) of x.
__device__ __forceinline__ uint32_t vcode_pair(uint32_t x, int nb) {
  const uint32_t y = (nb <= 2) ? (x << (5 - 2 * nb)) : (x >> (2 * nb - 5));
  return (y & 0x00600060u) | 0x3F803F80u;
}

typedef float v2f_t __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf_t __attribute__((ext_vector_type(2)));

// Two floats -> packed bf16 pair, round to nearest even (one v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((v2f_t){a, b}, v2bf_t));
}

// w ~= hi + lo with hi = bf16(w), lo = bf16(w - hi): relative error <= 2^-18, unbiased.
__device__ __forceinline__ void split_bf16(const float w[4], uint32_t& h01, uint32_t& h23,
                                           uint32_t& l01, uint32_t& l23) {
  h01 = pack_bf16(w[0], w[1]);
  h23 = pack_bf16(w[2], w[3]);
  l01 = pack_bf16(w[0] - __uint_as_float(h01 << 16), w[1] - __uint_as_float(h01 & 0xFFFF0000u));
  l23 = pack_bf16(w[2] - __uint_as_float(h23 << 16), w[3] - __uint_as_float(h23 & 0xFFFF0000u));
}

// ------------------------------------------------------------------ BF16 sink/window split

// Positions [0, n_sink) and [L - n_win, L) from the BF16 store; fp32 math, one wavefront per
// (KV head, sequence); writes the last split slot.  grid (Hkv, batch), block 64.
__global__ __launch_bounds__(64) void window_kernel(CacheGeom g, const uint16_t* __restrict__ sinkwin,
                                                  const int32_t* __restrict__ slot_ids, int hq,
                                                  const int32_t* __restrict__ seq_lens,
                                                  float sm_scale, Workspace ws) {
  const int lane = threadIdx.x;
  const int h = blockIdx.x, b = blockIdx.y;
  const int G = hq / g.hkv;
  const int L = max(seq_lens[b], 0);
  const int slot = slot_ids ? slot_ids[b] : b;
  const float sm_log2 = sm_scale * kLog2e;
  const int out_slot = ws.nslots - 1;
  __shared__ float s_q[8][kHeadDim];
  __shared__ float s_p[kMaxSinkWindow][8];
  const int n_sink = min(L, g.num_sink);
  const int n_win = min(g.window, L - n_sink);
  const int n = n_sink + n_win;
  for (int i = lane; i < G * kHeadDim; i += 64)
    s_q[i / kHeadDim][i % kHeadDim] =
        reinterpret_cast<const float*>(ws.qblock(b, hq, h * G + i / kHeadDim))[i % kHeadDim];
  __syncthreads();
  const bool slot_ok = sinkwin != nullptr && slot >= 0 && slot < g.num_slots;
  const size_t base = ((size_t)slot * g.hkv + h) * (size_t)(g.num_sink + g.window);
  float mloc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) mloc[j] = kNegBig;
  for (int t0 = 0; t0 < n; t0 += 64) {
    const int t = t0 + lane;
    if (t < n && slot_ok) {
      const int p = t < n_sink ? t : L - n_win + (t - n_sink);
      const int row = p < g.num_sink ? p : g.num_sink + p % g.window;
      const uint4* krow = reinterpret_cast<const uint4*>(sinkwin + (base + row) * 2 * kHeadDim);
      float dot[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) dot[j] = 0.f;
      for (int c8 = 0; c8 < kHeadDim / 8; ++c8) {
        const uint4 kk = krow[c8];
        const uint32_t w[4] = {kk.x, kk.y, kk.z, kk.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float k0 = __uint_as_float(w[e] << 16), k1 = __uint_as_float(w[e] & 0xFFFF0000u);
#pragma unroll
          for (int j = 0; j < 8; ++j)
            if (j < G) dot[j] = fmaf(s_q[j][8 * c8 + 2 * e + 1], k1,
                                     fmaf(s_q[j][8 * c8 + 2 * e], k0, dot[j]));
        }
      }
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (j < G) {
          s_p[t][j] = dot[j] * sm_log2;
          mloc[j] = fmaxf(mloc[j], dot[j] * sm_log2);
        }
    }
  }
  float m[8], l[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    float x = mloc[j];
    for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
    m[j] = x;
    l[j] = 0.f;
  }
  __syncthreads();
  for (int t0 = 0; t0 < n; t0 += 64) {
    const int t = t0 + lane;
    if (t < n && slot_ok) {
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (j < G) {
          const float p = __builtin_amdgcn_exp2f(s_p[t][j] - m[j]);
          s_p[t][j] = p;
          l[j] += p;
        }
    }
  }
#pragma unroll
  for (int j = 0; j < 8; ++j)
    for (int o = 32; o >= 1; o >>= 1) l[j] += __shfl_xor(l[j], o);
  __syncthreads();
  // P.V: lane -> channels 2*lane, 2*lane+1
  float o0[8], o1[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) o0[j] = o1[j] = 0.f;
  if (slot_ok) {
    for (int t = 0; t < n; ++t) {
      const int p = t < n_sink ? t : L - n_win + (t - n_sink);
      const int row = p < g.num_sink ? p : g.num_sink + p % g.window;
      const uint32_t vv =
          reinterpret_cast<const uint32_t*>(sinkwin + (base + row) * 2 * kHeadDim + kHeadDim)[lane];
      const float v0 = __uint_as_float(vv << 16), v1 = __uint_as_float(vv & 0xFFFF0000u);
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (j < G) {
          o0[j] = fmaf(s_p[t][j], v0, o0[j]);
          o1[j] = fmaf(s_p[t][j], v1, o1[j]);
        }
    }
  }
  for (int j = 0; j < G; ++j) {
    float* o = ws.o(b, hq, h * G + j, out_slot);
    const bool live = slot_ok && n > 0;
    reinterpret_cast<float2*>(o)[lane] = live ? make_float2(o0[j], o1[j]) : make_float2(0.f, 0.f);
    if (lane == 0)
      *ws.ml(b, hq, h * G + j, out_slot) = live ? make_float2(m[j], l[j]) : make_float2(kNegBig, 0.f);
  }
}

// ------------------------------------------------------------------------ INT2 page splits

// Lane-uniform helpers.
__device__ __forceinline__ float dpp_add_xor1(float x) {  // x + x[lane ^ 1] within quads
  return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, true));
}
__device__ __forceinline__ float dpp_add_xor2(float x) {  // x + x[lane ^ 2] within quads
  return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, true));
}
// max over lanes l, l^16, l^32, l^48 (the four 16-lane rows), without LDS.
__device__ __forceinline__ float rowmax4(float x) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float rowsum4(float x) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// (x & mask) | magic.  With mask in an SGPR and magic in a VGPR (see int2_decode_kernel) the
// compiler selects one v_and_or_b32; with both as literals it needs two instructions.
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t mask, uint32_t magic) {
  return (x & mask) | magic;
}

__device__ __forceinline__ float f16lo(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFF));
}
__device__ __forceinline__ float f16hi(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

struct PageRegs {
  uint2 kc;  // K code dwords of this lane (words kq and 4 + kq of token c16)
  uint2 vc;  // V code chunk of this lane (4 tokens x 8 channel blocks)
  uint4 km;  // K (scale, zero) of tokens 4*kq .. 4*kq+3, this lane's group
  uint4 vm;  // V (scale, zero), same tokens and group
};

constexpr int kTile = 1;  // pages per online-softmax step

template <int NCB>
struct SplitState {
  v4f acc[NCB][8];   // P.V accumulators: rows (query head 4*cb + kq, group i), cols 16*nb + c16
  float mrun[NCB];   // running max (log2 units) of this lane's query head
  float lsum[NCB];   // sum of p over this lane's tokens
  float zsum[NCB];   // sum of p * (zero_v - 4 * scale_v) over this lane's tokens
};

template <int NCB>
struct QOperands {
  v4i hi[NCB][2], lo[NCB][2];
  float qsum_s[NCB];  // (sum of q' over the lane's group) * 254 / qsc
  float cscale[NCB];  // qsc / 254 * sm_scale * log2(e)
};

// One tile of kTile pages: logits on the int8 MFMA, online softmax, P.V on the bf16 MFMA.
// MASKED: some tokens of the tile are outside the INT2 range [lo, hi) (or on a skipped page);
// their bytes may be stale, so every use is a select, never a multiply.
template <int NCB, bool MASKED>
__device__ __forceinline__ void int2_tile(const PageRegs (&d)[kTile], int pg, int lo, int hi,
                                          uint32_t live_pages, const QOperands<NCB>& qo,
                                          SplitState<NCB>& st, int kq, uint32_t vmask,
                                          uint32_t magic) {
  float lg[kTile][NCB][4];
  float tmax[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) tmax[cb] = -INFINITY;
#pragma unroll
  for (int u = 0; u < kTile; ++u) {
    const uint32_t w0 = d[u].kc.x, w1 = d[u].kc.y;
    const v4i ka0 = (v4i){(int)(w0 & 0x03030303u), (int)((w0 >> 2) & 0x03030303u),
                          (int)((w0 >> 4) & 0x03030303u), (int)((w0 >> 6) & 0x03030303u)};
    const v4i ka1 = (v4i){(int)(w1 & 0x03030303u), (int)((w1 >> 2) & 0x03030303u),
                          (int)((w1 >> 4) & 0x03030303u), (int)((w1 >> 6) & 0x03030303u)};
    const uint32_t kmw[4] = {d[u].km.x, d[u].km.y, d[u].km.z, d[u].km.w};
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      v4i dh = {0, 0, 0, 0}, dl = {0, 0, 0, 0};
      dh = __builtin_amdgcn_mfma_i32_16x16x64_i8(ka0, qo.hi[cb][0], dh, 0, 0, 0);
      dh = __builtin_amdgcn_mfma_i32_16x16x64_i8(ka1, qo.hi[cb][1], dh, 0, 0, 0);
      dl = __builtin_amdgcn_mfma_i32_16x16x64_i8(ka0, qo.lo[cb][0], dl, 0, 0, 0);
      dl = __builtin_amdgcn_mfma_i32_16x16x64_i8(ka1, qo.lo[cb][1], dl, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int dint = __mul24(dh[i], 254) + dl[i];
        float part = fmaf(f16lo(kmw[i]), (float)dint, f16hi(kmw[i]) * qo.qsum_s[cb]);
        part = dpp_add_xor1(part);
        part = dpp_add_xor2(part);
        float l2 = part * qo.cscale[cb];
        if (MASKED) {
          const int pos = (pg + u) * kPage + 4 * kq + i;
          const bool live = ((live_pages >> u) & 1u) && pos >= lo && pos < hi;
          l2 = live ? l2 : -INFINITY;
        }
        lg[u][cb][i] = l2;
        tmax[cb] = fmaxf(tmax[cb], l2);
      }
    }
  }

  // Online softmax: exact running max per query head, lazy rescale of the accumulators.
  bool need = false;
  float mnew[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    mnew[cb] = fmaxf(st.mrun[cb], rowmax4(tmax[cb]));
    need |= mnew[cb] > st.mrun[cb];
  }
  if (__any(need)) {
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      const float alpha = __builtin_amdgcn_exp2f(st.mrun[cb] - mnew[cb]);
      // accumulator rows belong to query head 4*cb + kq: its alpha sits in lane 4*kq
      const float arow = __shfl(alpha, 4 * kq);
      st.lsum[cb] *= alpha;
      st.zsum[cb] *= alpha;
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) st.acc[cb][nb] *= arow;
      st.mrun[cb] = mnew[cb];
    }
  }

#pragma unroll
  for (int u = 0; u < kTile; ++u) {
    // V codes -> bf16 (1 + code/4); pair nb of dword x holds codes at bits 2nb and 16 + 2nb.
    v4s vb[8];
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
      const uint32_t x0 = d[u].vc.x, x1 = d[u].vc.y;
      const uint32_t y0 = nb <= 2 ? (x0 << (5 - 2 * nb)) : (x0 >> (2 * nb - 5));
      const uint32_t y1 = nb <= 2 ? (x1 << (5 - 2 * nb)) : (x1 >> (2 * nb - 5));
      const uint32_t p0 = and_or(y0, vmask, magic), p1 = and_or(y1, vmask, magic);
      vb[nb] = __builtin_bit_cast(v4s, make_uint2(p0, p1));
    }
    const uint32_t vmw[4] = {d[u].vm.x, d[u].vm.y, d[u].vm.z, d[u].vm.w};
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      float w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = __builtin_amdgcn_exp2f(lg[u][cb][i] - st.mrun[cb]);
        const float sv = f16lo(vmw[i]), zv = f16hi(vmw[i]);
        const float zz = fmaf(-4.0f, sv, zv);
        if (MASKED) {
          const bool live = lg[u][cb][i] != -INFINITY;
          st.lsum[cb] += p;  // p == 0 exactly for masked tokens
          st.zsum[cb] = live ? fmaf(p, zz, st.zsum[cb]) : st.zsum[cb];
          w[i] = live ? p * sv : 0.f;
        } else {
          st.lsum[cb] += p;
          st.zsum[cb] = fmaf(p, zz, st.zsum[cb]);
          w[i] = p * sv;
        }
      }
      uint32_t h01, h23, l01, l23;
      split_bf16(w, h01, h23, l01, l23);
      const v4s ahi = __builtin_bit_cast(v4s, make_uint2(h01, h23));
      const v4s alo = __builtin_bit_cast(v4s, make_uint2(l01, l23));
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) {
        st.acc[cb][nb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ahi, vb[nb], st.acc[cb][nb], 0, 0, 0);
        st.acc[cb][nb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(alo, vb[nb], st.acc[cb][nb], 0, 0, 0);
      }
    }
  }
}

// NCB = number of 16-wide column blocks of (query head, group) pairs = ceil(G / 4).
// grid (max_splits, Hkv, batch), block 64: one wavefront per (split, KV head, sequence).
template <int NCB>
__global__ __launch_bounds__(64) void int2_decode_kernel(
    CacheGeom g, const uint8_t* __restrict__ pages, const int32_t* __restrict__ block_table,
    int hq, const int32_t* __restrict__ seq_lens, float sm_scale, int split_pages, Workspace ws) {
  const int lane = threadIdx.x;
  const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int max_splits = ws.nslots - 1;
  const int G = hq / g.hkv;
  const int L = max(seq_lens[b], 0);
  const float sm_log2 = sm_scale * kLog2e;
  const int kq = lane >> 4, c16 = lane & 15;
  const int grp = c16 & 3;  // quantisation group of this lane's (query head, group) column

  // INT2 positions [lo, hi) and this split's logical pages [pg0, pg1).
  const int n_sink = min(L, g.num_sink);
  const int n_win = min(g.window, L - n_sink);
  const int lo = n_sink, hi = L - n_win;
  int pg0 = split * split_pages;
  int pg1 = (split == max_splits - 1) ? 0x7fffffff : pg0 + split_pages;
  pg0 = max(pg0, lo / kPage);
  pg1 = min(min(pg1, (hi + kPage - 1) / kPage), g.max_pages);
  if (hi <= lo) pg1 = pg0;

  QOperands<NCB> qo;
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    const int j = 4 * cb + (c16 >> 2);
    const bool jvalid = j < G;
    const char* blk = ws.qblock(b, hq, h * G + (jvalid ? j : 0));
    const float qsc = *reinterpret_cast<const float*>(blk + kQScOff);
    const float qs = reinterpret_cast<const float*>(blk + kQSumOff)[grp];
    qo.qsum_s[cb] = qsc > 0.f ? qs * 254.0f / qsc : 0.f;
    // strictly positive so that a masked -inf logit never becomes 0 * inf
    qo.cscale[cb] = fmaxf(qsc / 254.0f * sm_log2, 1e-30f);
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int d = 4 * m + kq;  // 16-channel word of this lane's K quarter
      const bool use = jvalid && (d >> 1) == grp;
      const v4i zh = *reinterpret_cast<const v4i*>(blk + kQHiOff + 16 * d);
      const v4i zl = *reinterpret_cast<const v4i*>(blk + kQLoOff + 16 * d);
      const v4i zero = {0, 0, 0, 0};
      qo.hi[cb][m] = use ? zh : zero;
      qo.lo[cb][m] = use ? zl : zero;
    }
  }

  SplitState<NCB> st;
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) st.acc[cb][nb] = (v4f){0.f, 0.f, 0.f, 0.f};
    st.mrun[cb] = kNegBig;
    st.lsum[cb] = 0.f;
    st.zsum[cb] = 0.f;
  }
  // Opaque copies of the two V-code constants: mask in an SGPR, magic in a VGPR, so every
  // (x & mask) | magic is one instruction.  The empty asm statements emit nothing.
  uint32_t vmask = 0x00600060u, magic = 0x3F803F80u;
  asm volatile("" : "+s"(vmask));
  asm volatile("" : "+v"(magic));

  // Page ids of the split, 64 per lane register, fetched lane-parallel and read back per page
  // with v_readlane (no scalar-load latency inside the loop).
  const int32_t* bt = block_table + (size_t)b * g.max_pages;
  int id_base = pg0;
  int ids = (pg0 + lane < pg1) ? bt[pg0 + lane] : -1;

  auto page_id = [&](int pg) -> int {  // uniform
    if (pg >= pg1) return -1;
    if (pg - id_base >= 64) {
      id_base = pg;
      ids = (pg + lane < pg1) ? bt[pg + lane] : -1;
    }
    return __builtin_amdgcn_readlane(ids, pg - id_base);
  };
  auto load_tile = [&](int pgt, PageRegs (&d)[kTile], uint32_t& live) {
    live = 0;
#pragma unroll
    for (int u = 0; u < kTile; ++u) {
      const int page = page_id(pgt + u);
      if (page >= 0 && page < g.num_pages) {
        const uint8_t* rec = pages + ((size_t)page * g.hkv + h) * kRecord;
        d[u].kc = reinterpret_cast<const uint2*>(rec + kKCodes)[lane];
        d[u].vc = reinterpret_cast<const uint2*>(rec + kVCodes)[lane];
        d[u].km = *reinterpret_cast<const uint4*>(rec + kKMeta + 64 * grp + 16 * kq);
        d[u].vm = *reinterpret_cast<const uint4*>(rec + kVMeta + 64 * grp + 16 * kq);
        live |= 1u << u;
      } else {
        d[u].kc = make_uint2(0, 0);
        d[u].vc = make_uint2(0, 0);
        d[u].km = make_uint4(0, 0, 0, 0);
        d[u].vm = make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto run_tile = [&](int pgt, const PageRegs (&d)[kTile], uint32_t live) {
    const bool interior = live == (1u << kTile) - 1 && pgt * kPage >= lo &&
                          (pgt + kTile) * kPage <= hi;
    if (interior)
      int2_tile<NCB, false>(d, pgt, lo, hi, live, qo, st, kq, vmask, magic);
    else
      int2_tile<NCB, true>(d, pgt, lo, hi, live, qo, st, kq, vmask, magic);
  };

  // Two register buffers: the next tile's loads are in flight while the current one computes.
  PageRegs bufA[kTile], bufB[kTile];
  uint32_t liveA = 0, liveB = 0;
  int pg = pg0;
  if (pg < pg1) load_tile(pg, bufA, liveA);
  while (pg < pg1) {
    const int nxt = pg + kTile;
    if (nxt < pg1) load_tile(nxt, bufB, liveB);
    run_tile(pg, bufA, liveA);
    pg = nxt;
    if (pg >= pg1) break;
    const int nxt2 = pg + kTile;
    if (nxt2 < pg1) load_tile(nxt2, bufA, liveA);
    run_tile(pg, bufB, liveB);
    pg = nxt2;
  }

  // Finish: reduce l and the zero-point term over the four token quarters, assemble
  // o'[j][c] = 4 * acc[row (j, g(c))][c] + Z[j][g(c)], write the split's partials.
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    const float lt = rowsum4(st.lsum[cb]);
    const float zt = rowsum4(st.zsum[cb]);
    const int j = 4 * cb + kq;  // query head of the accumulator rows this lane holds
    float zrow[4];
#pragma unroll
    for (int gg = 0; gg < 4; ++gg) zrow[gg] = __shfl(zt, 4 * kq + gg);
    if (j < G) {
      float* o = ws.o(b, hq, h * G + j, split);
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) {
        const int gsel = nb >> 1;
        o[16 * nb + c16] = 4.0f * st.acc[cb][nb][gsel] + zrow[gsel];
      }
    }
    const float lrow = __shfl(lt, 4 * kq);
    const float mrow = __shfl(st.mrun[cb], 4 * kq);
    if (c16 == 0 && j < G) *ws.ml(b, hq, h * G + j, split) = make_float2(mrow, lrow);
  }
}

}  // namespace

hipError_t launch_decode(const CacheGeom& g, const uint8_t* pages, const uint16_t* sinkwin,
                         const int32_t* block_table, const int32_t* slot_ids, int batch,
                         int hq, const uint16_t* q, const int32_t* seq_lens, const float* rot_k,
                         float sm_scale, int split_pages, const Workspace& ws,
                         hipStream_t stream) {
  if (batch == 0) return hipSuccess;
  hipLaunchKernelGGL(q_prep_kernel, dim3(g.hkv, batch), dim3(128), 0, stream, q, rot_k, hq,
                     g.hkv, ws);
  const int G = hq / g.hkv;
  dim3 grid(ws.nslots - 1, g.hkv, batch);
  if (G <= 4)
    hipLaunchKernelGGL(int2_decode_kernel<1>, grid, dim3(64), 0, stream, g, pages, block_table,
                       hq, seq_lens, sm_scale, split_pages, ws);
  else
    hipLaunchKernelGGL(int2_decode_kernel<2>, grid, dim3(64), 0, stream, g, pages, block_table,
                       hq, seq_lens, sm_scale, split_pages, ws);
  hipLaunchKernelGGL(window_kernel, dim3(g.hkv, batch), dim3(64), 0, stream, g, sinkwin,
                     slot_ids, hq, seq_lens, sm_scale, ws);
  return hipGetLastError();
}

}  // namespace oscar
