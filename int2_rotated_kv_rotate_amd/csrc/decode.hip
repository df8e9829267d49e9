// Mixed-precision paged decode attention over the rotated INT2 cache.
//
// Method: OSCAR project card "FutureMLS-Lab/OSCAR", section "How it works" (BF16 sinks + BF16
// recent window + INT2 bulk, fused mixed-precision flash attention); OSCAR paper, "Abstract"
// (INT2 attention kernel that keeps the paged KV-cache layout; speed comes from reading fewer
// bytes).  Attention is computed in the rotated frame: q' = q . R_K makes q'.k' = q.k for
// orthogonal R_K, and the rotated output is rotated back with R_V^T by the combine kernel.
//
// Kernels
//   prep_window_kernel per (KV head, sequence): q' = q . R_K for the G query heads of the group
//                      plus an integer form of q' for the int8 matrix cores, and attention
//                      over the BF16 sink + window positions (the last split).
//   int2_decode_kernel per (split, KV head, sequence), one wavefront: walks the split's pages
//                      through the block table.  Per page it reads one 1536-byte record with
//                      four coalesced vector loads per lane, computes the G x 16 logits on the
//                      int8 MFMA (codes are exact int8, q' is two int8 pieces), runs the online
//                      softmax, and accumulates P.V on the bf16 MFMA (codes exact as bf16
//                      1 + code/4, weights p*scale as two bf16 pieces).
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

// ---------------------------------------------------------------- q rotation + BF16 window

// One workgroup (256 threads) per (KV head, sequence):
//  1. q' = q . R_K for the G query heads of the group (fp32), written to the workspace with its
//     int8 form for the matrix cores: q' ~= qsc * (hi + lo / 254), hi/lo in [-127, 127], stored
//     in MFMA slot order, plus the sum of q' over each 32-channel group;
//  2. attention over the BF16 positions [0, n_sink) and [L - n_win, L) (sinks + recent window,
//     rotated frame), written as the last split's partials (m in log2 units, l, o').
// Every global load is issued before its first use: R_K as 16 independent float4 loads per
// thread (partial sums over 16 input rows, reduced through LDS), each token's K row straight
// into the registers of the thread that scores it, and the V rows bulk-copied into LDS, so
// each phase pays about one memory latency.
constexpr int kPrepThreads = 256;

struct PrepPhase1 {
  float4 part[8][8][kHeadDim / 4];  // [input block][head][channel quad] partial q'
};
struct PrepPhase2 {
  float p[kMaxSinkWindow][8];       // logits, then probabilities
  float o[2][8][kHeadDim];          // P.V halves
};

__global__ __launch_bounds__(kPrepThreads) void prep_window_kernel(
    CacheGeom g, const uint16_t* __restrict__ q, const float* __restrict__ rot_k,
    const uint16_t* __restrict__ sinkwin, const int32_t* __restrict__ slot_ids, int hq,
    const int32_t* __restrict__ seq_lens, float sm_scale, Workspace ws) {
  const int h = blockIdx.x, b = blockIdx.y, t = threadIdx.x;
  const int lane = t & 63, wv = t >> 6;
  const int G = hq / g.hkv;
  extern __shared__ uint32_t s_v[];                    // [n][64] window V rows (bf16 pairs)
  __shared__ float s_q[8][kHeadDim];                   // q (bf16 widened)
  __shared__ float s_qr[8][kHeadDim];                  // q' = q . R_K
  __shared__ union { PrepPhase1 a; PrepPhase2 c; } s_u;
  __shared__ float s_red[4][8];

  const int L = max(seq_lens[b], 0);
  const int slot = slot_ids ? slot_ids[b] : b;
  const int n_sink = min(L, g.num_sink);
  const int n_win = min(g.window, L - n_sink);
  const bool live = sinkwin != nullptr && slot >= 0 && slot < g.num_slots && n_sink + n_win > 0;
  const int n = live ? n_sink + n_win : 0;
  const size_t base = ((size_t)slot * g.hkv + h) * (size_t)(g.num_sink + g.window);
  auto row_of = [&](int i) {  // window token index -> store row
    const int p = i < n_sink ? i : L - n_win + (i - n_sink);
    return p < g.num_sink ? p : g.num_sink + p % g.window;
  };

  // Issue the R_K loads: thread -> channel quad c4 = t % 32, input block ib = t / 32 (16 rows).
  const int c4 = t & 31, ib = t >> 5;
  const float4* R4 = reinterpret_cast<const float4*>(rot_k + (size_t)h * kHeadDim * kHeadDim);
  float4 r[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) r[k] = R4[(16 * ib + k) * (kHeadDim / 4) + c4];
  // This thread's window token: its K row into registers.
  uint4 kk[16];
  if (t < n) {
    const uint4* krow = reinterpret_cast<const uint4*>(sinkwin + (base + row_of(t)) * 2 * kHeadDim);
#pragma unroll
    for (int c8 = 0; c8 < 16; ++c8) kk[c8] = krow[c8];
  }
  // V rows into LDS.
  for (int e = t; e < n * (kHeadDim / 8); e += kPrepThreads) {
    const int i = e >> 4, w = e & 15;
    reinterpret_cast<uint4*>(s_v)[e] =
        reinterpret_cast<const uint4*>(sinkwin + (base + row_of(i)) * 2 * kHeadDim + kHeadDim)[w];
  }
  for (int i = t; i < G * kHeadDim; i += kPrepThreads)
    s_q[i / kHeadDim][i % kHeadDim] = bf16_to_f32(q[((size_t)b * hq + h * G) * kHeadDim + i]);
  __syncthreads();

  // 1. q' partial sums over this thread's 16 input rows, then reduce the 8 blocks in order.
  {
    float4 acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int i = 16 * ib + k;
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (j < G) {
          const float qi = s_q[j][i];
          acc[j].x = fmaf(qi, r[k].x, acc[j].x);
          acc[j].y = fmaf(qi, r[k].y, acc[j].y);
          acc[j].z = fmaf(qi, r[k].z, acc[j].z);
          acc[j].w = fmaf(qi, r[k].w, acc[j].w);
        }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (j < G) s_u.a.part[ib][j][c4] = acc[j];
  }
  __syncthreads();
  for (int e = t; e < G * kHeadDim; e += kPrepThreads) {
    const int j = e / kHeadDim, c = e % kHeadDim;
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) s += reinterpret_cast<const float*>(&s_u.a.part[k][j][0])[c];
    s_qr[j][c] = s;
  }
  __syncthreads();

  // int8 form: wave wv handles heads wv, wv + 4; lane -> channels 2*lane, 2*lane + 1.
  for (int j = wv; j < G; j += 4) {
    const float v0 = s_qr[j][2 * lane], v1 = s_qr[j][2 * lane + 1];
    float a = fmaxf(fabsf(v0), fabsf(v1));
    for (int o = 32; o >= 1; o >>= 1) a = fmaxf(a, __shfl_xor(a, o));
    float s = v0 + v1;  // 16 lanes = one 32-channel group
    for (int o = 8; o >= 1; o >>= 1) s += __shfl_xor(s, o);
    const float qsc = a / 127.0f;
    char* blk = ws.qblock(b, hq, h * G + j);
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int c = 2 * lane + e;
      const float v = e ? v1 : v0;
      int hi = 0, lo = 0;
      if (qsc > 0.f) {
        hi = max(-127, min(127, (int)__builtin_rintf(v / qsc)));
        lo = max(-127, min(127, (int)__builtin_rintf((v - (float)hi * qsc) * 254.0f / qsc)));
      }
      // slot order inside each 16-channel word: slot 4*i + b holds channel 4*b + i
      const int pos = 16 * (c / 16) + 4 * (c % 4) + (c % 16) / 4;
      blk[kQHiOff + pos] = (char)hi;
      blk[kQLoOff + pos] = (char)lo;
    }
    reinterpret_cast<float2*>(blk)[lane] = make_float2(v0, v1);
    if (lane == 0) *reinterpret_cast<float*>(blk + kQScOff) = qsc;
    if ((lane & 15) == 0) reinterpret_cast<float*>(blk + kQSumOff)[lane >> 4] = s;
  }

  // 2. Window logits: thread t scores token t from its K row in registers.
  const float sm_log2 = sm_scale * kLog2e;
  float lg[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) lg[j] = -INFINITY;
  if (t < n) {
    float dot[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) dot[j] = 0.f;
#pragma unroll
    for (int c8 = 0; c8 < 16; ++c8) {
      const uint32_t w[4] = {kk[c8].x, kk[c8].y, kk[c8].z, kk[c8].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float k0 = __uint_as_float(w[e] << 16), k1 = __uint_as_float(w[e] & 0xFFFF0000u);
        const int c = 8 * c8 + 2 * e;
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (j < G) dot[j] = fmaf(s_qr[j][c + 1], k1, fmaf(s_qr[j][c], k0, dot[j]));
      }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (j < G) lg[j] = dot[j] * sm_log2;
  }
  float m[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    float x = lg[j];
    for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
    if (lane == 0) s_red[wv][j] = x;
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < 8; ++j)
    m[j] = fmaxf(fmaxf(s_red[0][j], s_red[1][j]), fmaxf(s_red[2][j], s_red[3][j]));
  __syncthreads();
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float p = t < n && j < G ? __builtin_amdgcn_exp2f(lg[j] - m[j]) : 0.f;
    if (t < n) s_u.c.p[t][j] = p;
    float x = p;
    for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
    if (lane == 0) s_red[wv][j] = x;
  }
  __syncthreads();
  // P.V: thread -> channel pair cp, token quarter tq.
  {
    const int cp = t & 63, tq = t >> 6;
    float o0[8], o1[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) o0[j] = o1[j] = 0.f;
    for (int i = tq; i < n; i += 4) {
      const uint32_t vv = s_v[i * (kHeadDim / 2) + cp];
      const float v0 = __uint_as_float(vv << 16), v1 = __uint_as_float(vv & 0xFFFF0000u);
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (j < G) {
          o0[j] = fmaf(s_u.c.p[i][j], v0, o0[j]);
          o1[j] = fmaf(s_u.c.p[i][j], v1, o1[j]);
        }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (j < G && tq >= 2) {
        s_u.c.o[tq - 2][j][2 * cp] = o0[j];
        s_u.c.o[tq - 2][j][2 * cp + 1] = o1[j];
      }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (j < G && tq < 2) {
        s_u.c.o[tq][j][2 * cp] += o0[j];
        s_u.c.o[tq][j][2 * cp + 1] += o1[j];
      }
    __syncthreads();
  }
  const int out_slot = ws.nslots - 1;
  for (int i = t; i < G * kHeadDim; i += kPrepThreads) {
    const int j = i / kHeadDim, c = i % kHeadDim;
    ws.o(b, hq, h * G + j, out_slot)[c] = s_u.c.o[0][j][c] + s_u.c.o[1][j][c];
  }
  if (t < G) {
    const float l = s_red[0][t] + s_red[1][t] + s_red[2][t] + s_red[3][t];
    *ws.ml(b, hq, h * G + t, out_slot) = n > 0 ? make_float2(m[t], l) : make_float2(kNegBig, 0.f);
  }
}

// ------------------------------------------------------------------------ INT2 page splits
//
// Lane roles (lane l, t = l % 16, r = l / 16):
//   QK   S[(j,g)][t] = Qmask[(j,g)][:] . Kcodes[t][:]  (int8 MFMA, K = 128 channels)
//        A = Qmask: lane holds row (j,g) = (4*cb + (l%16)/4, l%4), i.e. q' of head j on the
//            channels of group g and 0 elsewhere, channel words 4*m + r (m = 0, 1);
//        B = K codes of token t, the same channel words;
//        D: lane holds column t and rows 4*r + i, i.e. head j = 4*cb + r, groups i = 0..3.
//        So each lane owns one (head, token) with all four group partial dot products.
//   PV   O[(j,g)][c] = W[(j,g)][t'] . Vcodes[t'][c]    (bf16 MFMA, K = 16 tokens)
//        A = W = p * scale_v as a hi/lo bf16 pair: lane holds row (j,g) = l%16 and tokens
//            4*r .. 4*r+3, so the (head, token)-owned values are transposed through a small
//            per-wave LDS tile;
//        B = V codes as bf16 1 + code/4: lane holds channel 16*nb + t and tokens 4*r .. 4*r+3;
//        D: lane holds channel 16*nb + t, rows 4*r + i = (head 4*cb + r, group i); only the
//           row of the channel's own group (i = nb / 2) is used.

// Within each 16-lane row: reductions across the row with DPP (no LDS).
template <int CTRL>
__device__ __forceinline__ float dpp_c(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float row_max16(float x) {
  x = fmaxf(x, dpp_c<0xB1>(x));    // quad_perm [1,0,3,2]
  x = fmaxf(x, dpp_c<0x4E>(x));    // quad_perm [2,3,0,1]
  x = fmaxf(x, dpp_c<0x124>(x));   // row_ror:4
  x = fmaxf(x, dpp_c<0x128>(x));   // row_ror:8
  return x;
}
__device__ __forceinline__ float row_sum16(float x) {
  x += dpp_c<0xB1>(x);
  x += dpp_c<0x4E>(x);
  x += dpp_c<0x124>(x);
  x += dpp_c<0x128>(x);
  return x;
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


// ---- page ring in LDS, filled by direct-to-LDS loads -------------------------------------
//
// Each page record (1536 B) is copied into a per-wave LDS slot by two global_load_lds_dwordx4
// (64 lanes, then 32 lanes, 16 B each), several pages ahead of the page being computed, so that the memory
// latency is covered without holding the data in VGPRs.  These loads and the reads of a slot
// are issued as inline assembly with an explicit vmcnt wait per page: the compiler does not
// track them (it would otherwise wait for every outstanding direct-to-LDS load before any LDS
// access).  Loads the compiler does issue are only ever waited on more strictly as a result.

constexpr int kRing = 4;            // LDS slots per wave: 1 being computed + 3 in flight
constexpr int kAhead = kRing - 1;

__device__ __forceinline__ uint32_t lds_offset(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Copy the 1536-byte record at `rec` into the LDS slot at byte offset `slot`: lane l moves 16
// bytes to slot + 16 l (bytes [0, 1024) with all lanes, then [1024, 1536) with lanes 0..31).
__device__ __forceinline__ void dma_record(const uint8_t* rec, uint32_t slot, int lane) {
  const uint8_t* a0 = rec + 16 * lane;
  asm volatile(
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, off"
      :
      : "v"(a0), "s"(slot)
      : "memory", "m0");
  if (lane < 32) {
    const uint8_t* a1 = rec + 1024 + 16 * lane;
    asm volatile(
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %0, off"
        :
        : "v"(a1), "s"(slot + 1024u)
        : "memory", "m0");
  }
}

// Wait until at most 2*N direct-to-LDS page loads (N pages) are still outstanding.
template <int N>
__device__ __forceinline__ void wait_pages() {
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(2 * N) : "memory");
}
__device__ __forceinline__ void wait_pages_rt(int n) {  // n in [0, kAhead]
  switch (n) {
    case 0: wait_pages<0>(); break;
    case 1: wait_pages<1>(); break;
    case 2: wait_pages<2>(); break;
    default: wait_pages<3>(); break;
  }
}

struct PageRegs {
  uint2 kc;  // K code words r and 4 + r of token t
  uint2 vc;  // V code chunk of this lane (channel residue t, tokens 4r .. 4r+3, 8 blocks)
  uint4 km;  // K (scale, zero) of token t, groups 0..3
  uint4 vm;  // V (scale, zero) of token t, groups 0..3
};

// Read this lane's part of the record in LDS slot `slot`.
__device__ __forceinline__ PageRegs read_slot(uint32_t slot, int lane, int t) {
  PageRegs d;
  const uint32_t a8 = slot + 8 * lane, a16 = slot + 16 * t;
  asm volatile(
      "ds_read_b64 %0, %4\n\t"
      "ds_read_b64 %1, %4 offset:512\n\t"
      "ds_read_b128 %2, %5 offset:1024\n\t"
      "ds_read_b128 %3, %5 offset:1280\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(d.kc), "=&v"(d.vc), "=&v"(d.km), "=&v"(d.vm)
      : "v"(a8), "v"(a16)
      : "memory");
  return d;
}

template <int NCB>
struct SplitState {
  v4f acc[NCB][8];     // P.V accumulators
  float mref[NCB];     // reference max (log2 units) of this lane's head; p = 2^(z - mref)
  float mtrue[NCB];    // exact running max of this lane's head
  float lsum[NCB];     // sum of p over this lane's token positions
  float zsum[NCB][4];  // sum of p * (zero_v - 4 * scale_v) per group
};

template <int NCB>
struct QOperands {
  v4i hi[NCB][2], lo[NCB][2];   // A operands (masked q' pieces), channel halves m = 0, 1
  float qs[NCB][4];             // (sum of q' over group g) * 254 / qsc for this lane's head
  float cscale[NCB];            // qsc / 254 * sm_scale * log2(e), > 0
};

// Per-wave LDS tile for the W transpose: [cb][hi/lo][row (j,g)][token] bf16.
template <int NCB>
struct WTile {
  uint16_t w[NCB][2][16][kPage];
};

// A split keeps the first live page's max as its reference: later logits may exceed it, and
// p = 2^(z - mref) > 1 is fine in fp32/bf16 as long as z - mref stays below this margin.
// Beyond it the split is recomputed once with its exact max (never in the loop: no rescale).
constexpr float kRefMargin = 64.0f;

// One page.  `live` says whether this lane's token is an INT2 position of a valid page; a dead
// token's slot may hold stale bytes, so its logit is replaced by -inf and its V scale/zero by 0
// (selects, never arithmetic on the stale values), which makes all its contributions exactly 0.
template <int NCB>
__device__ __forceinline__ void int2_page(const PageRegs& d, bool live, const QOperands<NCB>& qo,
                                          SplitState<NCB>& st, WTile<NCB>& tile, int t, int r,
                                          uint32_t vmask, uint32_t magic, bool fixed_ref) {
  const v4i ka0 = (v4i){(int)(d.kc.x & 0x03030303u), (int)((d.kc.x >> 2) & 0x03030303u),
                        (int)((d.kc.x >> 4) & 0x03030303u), (int)((d.kc.x >> 6) & 0x03030303u)};
  const v4i ka1 = (v4i){(int)(d.kc.y & 0x03030303u), (int)((d.kc.y >> 2) & 0x03030303u),
                        (int)((d.kc.y >> 4) & 0x03030303u), (int)((d.kc.y >> 6) & 0x03030303u)};
  const uint32_t kmw[4] = {d.km.x, d.km.y, d.km.z, d.km.w};
  const uint32_t vmw[4] = {live ? d.vm.x : 0u, live ? d.vm.y : 0u, live ? d.vm.z : 0u,
                           live ? d.vm.w : 0u};

  float lg[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    v4i dh = {0, 0, 0, 0}, dl = {0, 0, 0, 0};
    dh = __builtin_amdgcn_mfma_i32_16x16x64_i8(qo.hi[cb][0], ka0, dh, 0, 0, 0);
    dh = __builtin_amdgcn_mfma_i32_16x16x64_i8(qo.hi[cb][1], ka1, dh, 0, 0, 0);
    dl = __builtin_amdgcn_mfma_i32_16x16x64_i8(qo.lo[cb][0], ka0, dl, 0, 0, 0);
    dl = __builtin_amdgcn_mfma_i32_16x16x64_i8(qo.lo[cb][1], ka1, dl, 0, 0, 0);
    float a = 0.f;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int dint = __mul24(dh[g], 254) + dl[g];
      a = fmaf(f16lo(kmw[g]), (float)dint, a);
      a = fmaf(f16hi(kmw[g]), qo.qs[cb][g], a);
    }
    lg[cb] = live ? a * qo.cscale[cb] : -INFINITY;
    // reference / exact max of the head (one 16-lane row); no accumulator is ever rescaled
    const float pm = row_max16(lg[cb]);
    st.mtrue[cb] = fmaxf(st.mtrue[cb], pm);
    if (!fixed_ref && st.mref[cb] == kNegBig) st.mref[cb] = fmaxf(pm, kNegBig);
  }

  // V codes -> bf16 (1 + code/4); pair nb of dword x holds codes at bits 2nb and 16 + 2nb.
  v4s vb[8];
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) {
    const uint32_t y0 = nb <= 2 ? (d.vc.x << (5 - 2 * nb)) : (d.vc.x >> (2 * nb - 5));
    const uint32_t y1 = nb <= 2 ? (d.vc.y << (5 - 2 * nb)) : (d.vc.y >> (2 * nb - 5));
    vb[nb] = __builtin_bit_cast(v4s, make_uint2(and_or(y0, vmask, magic), and_or(y1, vmask, magic)));
  }

#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    // p = 0 for masked tokens and until the split has a reference (exp2(-inf) = 0)
    const float p = __builtin_amdgcn_exp2f(lg[cb] - st.mref[cb]);
    st.lsum[cb] += p;
    float w[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const float sv = f16lo(vmw[g]), zv = f16hi(vmw[g]);
      st.zsum[cb][g] = fmaf(p, fmaf(-4.0f, sv, zv), st.zsum[cb][g]);
      w[g] = fmaf(p, sv, 0.0f);
    }
    uint32_t h01, h23, l01, l23;
    split_bf16(w, h01, h23, l01, l23);
    // transpose: this lane's (head r, token t, groups 0..3) -> rows 4r + g, column t
    const int row = 4 * r;
    tile.w[cb][0][row + 0][t] = (uint16_t)h01;
    tile.w[cb][0][row + 1][t] = (uint16_t)(h01 >> 16);
    tile.w[cb][0][row + 2][t] = (uint16_t)h23;
    tile.w[cb][0][row + 3][t] = (uint16_t)(h23 >> 16);
    tile.w[cb][1][row + 0][t] = (uint16_t)l01;
    tile.w[cb][1][row + 1][t] = (uint16_t)(l01 >> 16);
    tile.w[cb][1][row + 2][t] = (uint16_t)l23;
    tile.w[cb][1][row + 3][t] = (uint16_t)(l23 >> 16);
    // A operands: row (j,g) = l % 16 (= t as an index), tokens 4r .. 4r+3
    const v4s ahi = *reinterpret_cast<const v4s*>(&tile.w[cb][0][t][4 * r]);
    const v4s alo = *reinterpret_cast<const v4s*>(&tile.w[cb][1][t][4 * r]);
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
      st.acc[cb][nb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ahi, vb[nb], st.acc[cb][nb], 0, 0, 0);
      st.acc[cb][nb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(alo, vb[nb], st.acc[cb][nb], 0, 0, 0);
    }
  }
}

// NCB = number of 16-row blocks of (query head, group) pairs = ceil(G / 4).
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
  const int t = lane & 15, r = lane >> 4;
  __shared__ WTile<NCB> tile;
  __shared__ __attribute__((aligned(16))) uint8_t ring[kRing][kRecord];
  const uint32_t ring0 = lds_offset(&ring[0][0]);

  // INT2 positions [lo, hi) and this split's logical pages [pg0, pg1).
  const int n_sink = min(L, g.num_sink);
  const int n_win = min(g.window, L - n_sink);
  const int lo = n_sink, hi = L - n_win;
  int pg0 = split * split_pages;
  int pg1 = (split == max_splits - 1) ? 0x7fffffff : pg0 + split_pages;
  pg0 = max(pg0, lo / kPage);
  pg1 = min(min(pg1, (hi + kPage - 1) / kPage), g.max_pages);
  if (hi <= lo || g.num_pages < 1) pg1 = pg0;

  QOperands<NCB> qo;
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    // A-operand row of this lane: head 4*cb + t/4, group t%4
    const int ja = 4 * cb + (t >> 2), ga = t & 3;
    const char* blka = ws.qblock(b, hq, h * G + (ja < G ? ja : 0));
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int dw = 4 * m + r;  // 16-channel word of this lane's K quarter
      const bool use = ja < G && (dw >> 1) == ga;
      const v4i zh = *reinterpret_cast<const v4i*>(blka + kQHiOff + 16 * dw);
      const v4i zl = *reinterpret_cast<const v4i*>(blka + kQLoOff + 16 * dw);
      const v4i zero = {0, 0, 0, 0};
      qo.hi[cb][m] = use ? zh : zero;
      qo.lo[cb][m] = use ? zl : zero;
    }
    // D rows of this lane: head 4*cb + r
    const int jd = 4 * cb + r;
    const char* blkd = ws.qblock(b, hq, h * G + (jd < G ? jd : 0));
    const float qsc = jd < G ? *reinterpret_cast<const float*>(blkd + kQScOff) : 0.f;
#pragma unroll
    for (int gg = 0; gg < 4; ++gg)
      qo.qs[cb][gg] = qsc > 0.f ? reinterpret_cast<const float*>(blkd + kQSumOff)[gg] * 254.0f / qsc : 0.f;
    // strictly positive so that a masked -inf logit never becomes 0 * inf
    qo.cscale[cb] = fmaxf(qsc / 254.0f * sm_log2, 1e-30f);
  }

  // Opaque copies of the two V-code constants: mask in an SGPR, magic in a VGPR, so every
  // (x & mask) | magic is one instruction.  The empty asm statements emit nothing.
  uint32_t vmask = 0x00600060u, magic = 0x3F803F80u;
  asm volatile("" : "+s"(vmask));
  asm volatile("" : "+v"(magic));

  const int32_t* bt = block_table + (size_t)b * g.max_pages;
  const uint8_t* pages_h = pages + (size_t)h * kRecord;      // record of (page 0, head h)
  const size_t rec_stride = (size_t)g.hkv * kRecord;         // bytes between pages
  SplitState<NCB> st;
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    st.mref[cb] = kNegBig;
    st.mtrue[cb] = kNegBig;
  }
#pragma nounroll
  for (int pass = 0; pass < 2; ++pass) {
    const bool fixed_ref = pass > 0;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) st.acc[cb][nb] = (v4f){0.f, 0.f, 0.f, 0.f};
      st.lsum[cb] = 0.f;
#pragma unroll
      for (int gg = 0; gg < 4; ++gg) st.zsum[cb][gg] = 0.f;
    }

    // Page ids come from uniform (scalar) loads, fetched one iteration before they are used;
    // scalar loads are counted by lgkmcnt, so waiting for one never drains the page ring.
    auto load_id = [&](int pg) -> int { return pg < pg1 ? bt[pg] : -1; };
    // Every page in [pg0, pg1) issues exactly one record copy (a skipped page copies page 0 of
    // the pool and is masked), so the per-page wait counts are exact.
    uint32_t live_bits = 0;  // bit (pg % 32): page id valid
    auto issue = [&](int pg, int page) {
      const bool ok = page >= 0 && page < g.num_pages;
      const uint8_t* rec = pages_h + (size_t)(ok ? page : 0) * rec_stride;
      dma_record(rec, ring0 + (uint32_t)(pg & (kRing - 1)) * kRecord, lane);
      live_bits = ok ? (live_bits | (1u << (pg & 31))) : (live_bits & ~(1u << (pg & 31)));
    };

    for (int k = 0; k < kAhead; ++k)
      if (pg0 + k < pg1) issue(pg0 + k, load_id(pg0 + k));
    int id_next = load_id(pg0 + kAhead);
    for (int pg = pg0; pg < pg1; ++pg) {
      if (pg + kAhead < pg1) {
        issue(pg + kAhead, id_next);
        id_next = load_id(pg + kAhead + 1);
        wait_pages<kAhead>();
      } else {
        wait_pages_rt(pg1 - 1 - pg);
      }
      const PageRegs d = read_slot(ring0 + (uint32_t)(pg & (kRing - 1)) * kRecord, lane, t);
      const int pos = pg * kPage + t;
      const bool live = ((live_bits >> (pg & 31)) & 1u) && pos >= lo && pos < hi;
      int2_page<NCB>(d, live, qo, st, tile, t, r, vmask, magic, fixed_ref);
    }

    // A logit beyond the reference margin: recompute once with the exact max (rare path).
    bool redo = false;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) redo |= st.mtrue[cb] > st.mref[cb] + kRefMargin;
    if (pass > 0 || !__any(redo)) break;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) st.mref[cb] = st.mtrue[cb];
  }

  // Finish: l and the zero-point terms reduced over the row's 16 tokens; the accumulator row
  // of a lane (head 4*cb + r) matches its own row, so no exchange is needed.
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    const float lt = row_sum16(st.lsum[cb]);
    float zt[4];
#pragma unroll
    for (int gg = 0; gg < 4; ++gg) zt[gg] = row_sum16(st.zsum[cb][gg]);
    const int j = 4 * cb + r;
    if (j < G) {
      float* o = ws.o(b, hq, h * G + j, split);
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) o[16 * nb + t] = 4.0f * st.acc[cb][nb][nb >> 1] + zt[nb >> 1];
      if (t == 0) *ws.ml(b, hq, h * G + j, split) = make_float2(st.mref[cb], lt);
    }
  }
}

}  // namespace

hipError_t launch_decode(const CacheGeom& g, const uint8_t* pages, const uint16_t* sinkwin,
                         const int32_t* block_table, const int32_t* slot_ids, int batch,
                         int hq, const uint16_t* q, const int32_t* seq_lens, const float* rot_k,
                         float sm_scale, int split_pages, const Workspace& ws,
                         hipStream_t stream) {
  if (batch == 0) return hipSuccess;
  // dynamic LDS: the window rows of one (sequence, KV head)
  const size_t win_lds = (size_t)(g.num_sink + g.window) * kHeadDim * sizeof(uint16_t);
  hipLaunchKernelGGL(prep_window_kernel, dim3(g.hkv, batch), dim3(kPrepThreads), win_lds, stream,
                     g, q, rot_k, sinkwin, slot_ids, hq, seq_lens, sm_scale, ws);
  const int G = hq / g.hkv;
  dim3 grid(ws.nslots - 1, g.hkv, batch);
  if (G <= 4)
    hipLaunchKernelGGL(int2_decode_kernel<1>, grid, dim3(64), 0, stream, g, pages, block_table,
                       hq, seq_lens, sm_scale, split_pages, ws);
  else
    hipLaunchKernelGGL(int2_decode_kernel<2>, grid, dim3(64), 0, stream, g, pages, block_table,
                       hq, seq_lens, sm_scale, split_pages, ws);
  return hipGetLastError();
}

}  // namespace oscar
