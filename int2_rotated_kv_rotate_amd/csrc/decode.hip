// Mixed-precision paged decode attention over the rotated INT2 cache.
//
// Method: OSCAR project card "FutureMLS-Lab/OSCAR", section "How it works" (BF16 sinks + BF16
// recent window + INT2 bulk, fused mixed-precision flash attention); OSCAR paper, "Abstract"
// (INT2 attention kernel that keeps the paged KV-cache layout; speed comes from reading fewer
// bytes).  Attention is computed in the rotated frame: q' = q . R_K makes q'.k' = q.k for
// orthogonal R_K, and the rotated output is rotated back with R_V^T by the combine kernel.
//
// Kernels
//   prep_q_kernel      (step.hip) per (KV head, sequence): q' = q . R_K for the G query heads of
//                      the group plus an integer form of q' for the int8 matrix cores; one
//                      extra workgroup writes the work plan of the INT2 workers.
//   int2_decode_kernel persistent INT2 workers, one wavefront each: a worker walks an equal
//                      share of all pages of all (sequence, KV head) pairs through the block
//                      tables.  Per page it copies one 1536-byte record into an LDS ring with
//                      direct-to-LDS loads, computes the G x 16 logits on the int8 MFMA (codes
//                      are exact int8, q' is two int8 pieces), runs the softmax against a
//                      reference max, and accumulates P.V on the bf16 MFMA (codes exact as
//                      bf16 1 + code/16 or 1 + code/4, weights p*scale as two bf16 pieces).
//                      Extra workgroups at the end of the grid attend over each pair's BF16
//                      sink + window positions.
//
// MFMA operand layouts (16x16 tiles, wave64): an A operand row m lives in lane m + 16*k4 and a
// B operand column n in lane n + 16*k4, with k4 selecting a quarter of the K dimension; the
// 16x16 result puts rows 4*(lane/16) + i of column lane%16 in accumulator register i.  The K
// axis is permuted consistently on both operands, which leaves the product unchanged.
#include <atomic>

#include "oscar_internal.h"

namespace oscar {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegBig = -1.0e30f;

// ---------------------------------------------------------------------- small wave helpers

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


// ---- page-pair ring in LDS, filled by direct-to-LDS loads --------------------------------
//
// Pages are processed in pairs.  A pair's two records (1536 B each) are copied into a per-wave
// LDS pair slot of 3072 B by four global_load_lds_dwordx4 (16 B per lane): record A bytes
// [0, 1024) to [0, 1024), record B bytes [0, 1024) to [1024, 2048), and the two 512-byte tails
// to [2048, 2560) (lanes 0..31) and [2560, 3072) (lanes 32..63).  The next pair is in flight
// while one is computed, so the memory latency is covered without holding data in VGPRs.
// These loads and the reads of a slot are inline assembly with an explicit vmcnt wait per
// pair: the compiler does not track them (it would otherwise wait for every outstanding
// direct-to-LDS load before any LDS access).  Loads the compiler does issue are only ever
// waited on more strictly as a result.

constexpr int kPairBytes = 3 * 1024;
constexpr int kPairSlots = 2;  // the pair being computed + the next one in flight
constexpr int kRingBytes = kPairSlots * kPairBytes;
constexpr int kPairHeadB = 1024;   // record B head; the tails follow at 2048 and 2560

__device__ __forceinline__ uint32_t lds_offset(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Copy records recA and recB (uniform addresses) into the pair slot at LDS byte offset ps.
// Lane l's 16 bytes land at M0 + 16 l.  voff = 16 l reads the heads; the tails are copied by
// two half-wave loads (exec restricted inside the statement and restored before it ends) with
// per-lane offsets vta = 1024 + 16 l (lanes 0..31: A bytes [1024, 1536)) and vtb = 512 + 16 l
// (lanes 32..63: B bytes [1024, 1536)).  No immediate offsets are used.  The three M0 values
// are computed outside the statement, which contains no instruction that writes SCC: the
// compiler may keep a condition live in SCC across it.
__device__ __forceinline__ void dma_pair(const uint8_t* recA, const uint8_t* recB, uint32_t ps,
                                         uint32_t voff, uint32_t vta, uint32_t vtb) {
  uint64_t saved;
  const uint32_t ps1 = __builtin_amdgcn_readfirstlane(ps + 0x400u);
  const uint32_t ps2 = __builtin_amdgcn_readfirstlane(ps + 0x800u);
  asm volatile(
      "s_mov_b32 m0, %[ps]\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %[v], %[a]\n\t"
      "s_mov_b32 m0, %[ps1]\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %[v], %[b]\n\t"
      "s_mov_b32 m0, %[ps2]\n\t"
      "s_mov_b64 %[sv], exec\n\t"
      "s_mov_b32 exec_hi, 0\n\t"
      "global_load_lds_dwordx4 %[ta], %[a]\n\t"
      "s_mov_b64 exec, %[sv]\n\t"
      "s_mov_b32 exec_lo, 0\n\t"
      "global_load_lds_dwordx4 %[tb], %[b]\n\t"
      "s_mov_b64 exec, %[sv]"
      : [sv] "=&s"(saved)
      : [ps] "s"(ps), [ps1] "s"(ps1), [ps2] "s"(ps2), [v] "v"(voff), [ta] "v"(vta),
        [tb] "v"(vtb), [a] "s"(recA), [b] "s"(recB)
      : "memory", "m0");
}

// Wait until at most N pairs' copies (4 loads each) are still outstanding.
template <int N>
__device__ __forceinline__ void wait_pairs() {
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(4 * N) : "memory");
}

// This lane's K operands of page X of a pair: K code words r and 4 + r of token t, and the K
// (scale, zero) of token t for groups 0..3.
struct PageK {
  uint2 kc;
  uint4 km;
};
// V scale/zero of token t (page A, page B) and this lane's V code words for P.V: page kq / 2,
// token quads 2 (kq % 2) and 2 (kq % 2) + 1 of channel residue t (8 tokens of one channel).
struct PairV {
  uint4 vmA, vmB;
  uint4 vs;
};

// K parts of both pages of the pair slot at LDS offset ps.  a8 = 8 * lane, a16 = 16 * t.
__device__ __forceinline__ void read_pair_k(uint32_t ps, uint32_t a8, uint32_t a16, PageK& A,
                                            PageK& B) {
  asm volatile(
      "ds_read_b64 %0, %4\n\t"
      "ds_read_b64 %1, %4 offset:1024\n\t"
      "ds_read_b128 %2, %5 offset:2048\n\t"
      "ds_read_b128 %3, %5 offset:2560\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(A.kc), "=&v"(B.kc), "=&v"(A.km), "=&v"(B.km)
      : "v"(ps + a8), "v"(ps + a16)
      : "memory");
}
// V parts.  av = this lane's V code offset within a pair slot.
__device__ __forceinline__ void read_pair_v(uint32_t ps, uint32_t a16, uint32_t av, PairV& V) {
  asm volatile(
      "ds_read_b128 %0, %3 offset:2304\n\t"
      "ds_read_b128 %1, %3 offset:2816\n\t"
      "ds_read2_b64 %2, %4 offset1:16\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(V.vmA), "=&v"(V.vmB), "=&v"(V.vs)
      : "v"(ps + a16), "v"(ps + av)
      : "memory");
}

// Layouts of the 16 MFMA rows: NCB = 1 or 2 blocks of (query head, group) rows, 4 heads x 4
// groups each (G <= 4: one block; a lane owns one head per block); NCB = 8 (G = 8): rows
// (head, group pair), 8 heads x 2 groups, one block for groups {0, 1} and one for {2, 3}, so a
// QK product needs only the half of the channels that its groups cover and a P.V product uses
// 8 of its 16 rows; a lane owns two heads.
template <int NCB>
constexpr int kLaneHeads = NCB == 8 ? 2 : NCB;   // heads whose softmax state a lane keeps
template <int NCB>
constexpr int kAccSets = NCB == 8 ? 1 : NCB;     // sets of 8 column-block accumulators

template <int NCB>
struct SplitState {
  v4f acc[kAccSets<NCB>][8];  // P.V accumulators
  float mref[kLaneHeads<NCB>];    // reference (log2 units) of a lane head; p = 2^(z - mref)
  float mlane[kLaneHeads<NCB>];   // running max of a lane head's unscaled logits
  float lsum[kLaneHeads<NCB>];    // sum of p over this lane's token positions
  float zp[kLaneHeads<NCB>][4];   // sum of p * zero_v per group
  v4f wsum[kLaneHeads<NCB>];      // sums of the bf16 weights W = p * scale_v of each row of a
                                  // block (against a column of ones)
};

template <int NCB>
struct QOperands {
  v4i hi[NCB][2], lo[NCB][2];   // A operands (masked q' pieces), channel halves m = 0, 1
  float qs[NCB][4];             // sum over group g of the encoded q' (254*hi + lo), this lane's head
  float cscale[NCB];            // qsc / 254 * sm_scale * log2(e), > 0
};
template <>
struct QOperands<8> {
  v4i hi[2], lo[2];             // A operands of the two blocks (groups {0,1} on channel half 0,
                                // {2,3} on half 1), masked to the row's group
  float qs[2][4];               // group sums of the encoded q' of the lane's two heads
  float cscale[2];
};

// Per-wave LDS tile for the W transpose: [cb][hi/lo][row (j,g)][token of the pair] bf16, page A
// tokens in columns 0..15, page B in 16..31.  Rows hold 36 entries (72 bytes): the 16-lane
// groups of one write land on distinct banks and the 8-token A operand reads are 8-byte aligned.
constexpr int kTileRow = 36;
template <int NCB>
struct WTile {
  uint16_t w[kLaneHeads<NCB>][2][16][kTileRow];   // [block][hi/lo][row][token of the pair]
};

// A run keeps the first page's max as its reference: later logits may exceed it, and
// p = 2^(z - mref) > 1 is fine in fp32/bf16 as long as z - mref stays below this margin.
// Beyond it the run is recomputed once with its exact max (never in the loop: no rescale).
constexpr float kRefMargin = 64.0f;

// V code words -> B operands.  Column blocks nb = 2q and 2q + 1 (the two halves of group q)
// come from one shifted copy of each code word: block 2q's codes sit at bits 3-4 (and 19-20),
// read as bf16 1 + code/16, block 2q + 1's at bits 5-6 (and 21-22), read as 1 + code/4.
constexpr float kVScale[2] = {16.0f, 4.0f};  // code = scale * (bf16 value - 1), even / odd nb

// Logits of one page in units of cscale: sum_g s_g * (q'.codes)_g + z_g * (sum of q' over g).
// MASKED: tokens outside [lo, hi) may hold stale bytes and get -inf (a select, never arithmetic
// on the stale values).
template <int NCB, bool MASKED>
__device__ __forceinline__ void page_logits(const PageK& d, bool live, const QOperands<NCB>& qo,
                                            float a[kLaneHeads<NCB>]) {
  const v4i ka0 = (v4i){(int)(d.kc.x & 0x03030303u), (int)((d.kc.x >> 2) & 0x03030303u),
                        (int)((d.kc.x >> 4) & 0x03030303u), (int)((d.kc.x >> 6) & 0x03030303u)};
  const v4i ka1 = (v4i){(int)(d.kc.y & 0x03030303u), (int)((d.kc.y >> 2) & 0x03030303u),
                        (int)((d.kc.y >> 4) & 0x03030303u), (int)((d.kc.y >> 6) & 0x03030303u)};
  const uint32_t kmw[4] = {d.km.x, d.km.y, d.km.z, d.km.w};
  if constexpr (NCB == 8) {
    // D element i of a lane: head 2r + i/2, group i%2 (block A) or 2 + i%2 (block B)
    const v4i zero = {0, 0, 0, 0};
    const v4i dhA = __builtin_amdgcn_mfma_i32_16x16x64_i8(qo.hi[0], ka0, zero, 0, 0, 0);
    const v4i dlA = __builtin_amdgcn_mfma_i32_16x16x64_i8(qo.lo[0], ka0, zero, 0, 0, 0);
    const v4i dhB = __builtin_amdgcn_mfma_i32_16x16x64_i8(qo.hi[1], ka1, zero, 0, 0, 0);
    const v4i dlB = __builtin_amdgcn_mfma_i32_16x16x64_i8(qo.lo[1], ka1, zero, 0, 0, 0);
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      float x = 0.f;
#pragma unroll
      for (int gl = 0; gl < 2; ++gl) {
        const int i = 2 * hh + gl;
        const int dA = __mul24(dhA[i], 254) + dlA[i], dB = __mul24(dhB[i], 254) + dlB[i];
        x = fmaf(f16lo(kmw[gl]), (float)dA, x);
        x = fmaf(f16hi(kmw[gl]), qo.qs[hh][gl], x);
        x = fmaf(f16lo(kmw[2 + gl]), (float)dB, x);
        x = fmaf(f16hi(kmw[2 + gl]), qo.qs[hh][2 + gl], x);
      }
      if (MASKED) x = live ? x : -INFINITY;
      a[hh] = x;
    }
    return;
  } else {
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    v4i dh = {0, 0, 0, 0}, dl = {0, 0, 0, 0};
    dh = __builtin_amdgcn_mfma_i32_16x16x64_i8(qo.hi[cb][0], ka0, dh, 0, 0, 0);
    dh = __builtin_amdgcn_mfma_i32_16x16x64_i8(qo.hi[cb][1], ka1, dh, 0, 0, 0);
    dl = __builtin_amdgcn_mfma_i32_16x16x64_i8(qo.lo[cb][0], ka0, dl, 0, 0, 0);
    dl = __builtin_amdgcn_mfma_i32_16x16x64_i8(qo.lo[cb][1], ka1, dl, 0, 0, 0);
    float x = 0.f;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int dint = __mul24(dh[g], 254) + dl[g];
      x = fmaf(f16lo(kmw[g]), (float)dint, x);
      x = fmaf(f16hi(kmw[g]), qo.qs[cb][g], x);
    }
    if (MASKED) x = live ? x : -INFINITY;
    a[cb] = x;
  }
  }
}

// Softmax weights of one page and their transpose into the W tile (columns col0 + t):
// p = 2^(a * cscale - mref), W = p * scale_v as a bf16 pair (hi = W truncated, lo = the rest
// rounded to nearest even; relative error <= 2^-17, unbiased).  A dead token has p = 0 and its
// V scale/zero replaced by 0.
template <int NCB, bool MASKED>
__device__ __forceinline__ void page_weights(const float a[kLaneHeads<NCB>], uint4 vm, bool live,
                                             const QOperands<NCB>& qo, SplitState<NCB>& st,
                                             WTile<NCB>& tile, int t, int r, int col0) {
  uint32_t vmw[4] = {vm.x, vm.y, vm.z, vm.w};
  if (MASKED) {
#pragma unroll
    for (int g = 0; g < 4; ++g) vmw[g] = live ? vmw[g] : 0u;
  }
#pragma unroll
  for (int cb = 0; cb < kLaneHeads<NCB>; ++cb) {
    const float p = __builtin_amdgcn_exp2f(fmaf(a[cb], qo.cscale[cb], -st.mref[cb]));
    st.lsum[cb] += p;
    float w[4], lo[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const float sv = f16lo(vmw[g]), zv = f16hi(vmw[g]);
      w[g] = fmaf(p, sv, 0.0f);  // one v_fma_mix_f32 from the fp16 scale
      st.zp[cb][g] = fmaf(p, zv, st.zp[cb][g]);
      lo[g] = w[g] - __uint_as_float(__float_as_uint(w[g]) & 0xFFFF0000u);
    }
    const uint32_t l01 = pack_bf16(lo[0], lo[1]), l23 = pack_bf16(lo[2], lo[3]);
    const int col = col0 + t;
    if constexpr (NCB == 8) {
      // lane head cb = head 2r + cb: group g -> block g/2, row 2 (2r + cb) + g%2
      const int row = 4 * r + 2 * cb;
      const uint16_t lp[4] = {(uint16_t)l01, (uint16_t)(l01 >> 16), (uint16_t)l23, (uint16_t)(l23 >> 16)};
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        tile.w[g >> 1][0][row + (g & 1)][col] = (uint16_t)(__float_as_uint(w[g]) >> 16);
        tile.w[g >> 1][1][row + (g & 1)][col] = lp[g];
      }
      continue;
    }
    // transpose: this lane's (head r, token t, groups 0..3) -> rows 4r + g, column col0 + t
    const int row = 4 * r;
#pragma unroll
    for (int g = 0; g < 4; ++g) tile.w[cb][0][row + g][col] = (uint16_t)(__float_as_uint(w[g]) >> 16);
    tile.w[cb][1][row + 0][col] = (uint16_t)l01;
    tile.w[cb][1][row + 1][col] = (uint16_t)(l01 >> 16);
    tile.w[cb][1][row + 2][col] = (uint16_t)l23;
    tile.w[cb][1][row + 3][col] = (uint16_t)(l23 >> 16);
  }
}

// One pair of pages.  MASKED: either page may hold positions outside [lo, hi) (liveA/liveB per
// lane token).  FIRST: page A sets the run's reference max (unless a fixed reference is given).
// after_reads() runs once the pair's LDS reads have completed (the page-id prefetch goes there,
// so that waiting for those reads never waits for it).
template <int NCB, bool MASKED, bool FIRST, class AfterReads>
__device__ __forceinline__ void int2_pair(uint32_t ps, uint32_t a8, uint32_t a16, uint32_t av,
                                          bool liveA, bool liveB, const QOperands<NCB>& qo,
                                          SplitState<NCB>& st, WTile<NCB>& tile, int t, int r,
                                          uint32_t mask_e, uint32_t mask_o, uint32_t magic,
                                          v8bf ones, bool fixed_ref, AfterReads&& after_reads) {
  PageK kA, kB;
  read_pair_k(ps, a8, a16, kA, kB);
  float aA[kLaneHeads<NCB>], aB[kLaneHeads<NCB>];
  page_logits<NCB, MASKED>(kA, liveA, qo, aA);
  page_logits<NCB, MASKED>(kB, liveB, qo, aB);
#pragma unroll
  for (int cb = 0; cb < kLaneHeads<NCB>; ++cb) {
    st.mlane[cb] = fmaxf(st.mlane[cb], fmaxf(aA[cb], aB[cb]));
    if (FIRST && !fixed_ref) st.mref[cb] = fmaxf(row_max16(aA[cb]) * qo.cscale[cb], kNegBig);
  }
  PairV V;
  read_pair_v(ps, a16, av, V);
  after_reads();
  page_weights<NCB, MASKED>(aA, V.vmA, liveA, qo, st, tile, t, r, 0);
  page_weights<NCB, MASKED>(aB, V.vmB, liveB, qo, st, tile, t, r, kPage);

  const uint32_t vsw[4] = {V.vs.x, V.vs.y, V.vs.z, V.vs.w};
  // A operands of every column block: row (j,g) = l % 16 (= t as an index), tokens 8r .. 8r+7
  // of the pair (rows are 8-byte aligned only: two 8-byte reads each)
  v8bf ahi[kLaneHeads<NCB>], alo[kLaneHeads<NCB>];
#pragma unroll
  for (int cb = 0; cb < kLaneHeads<NCB>; ++cb) {
    const uint2* ph = reinterpret_cast<const uint2*>(&tile.w[cb][0][t][8 * r]);
    const uint2* pl = reinterpret_cast<const uint2*>(&tile.w[cb][1][t][8 * r]);
    const uint2 h0 = ph[0], h1 = ph[1], l0 = pl[0], l1 = pl[1];
    ahi[cb] = __builtin_bit_cast(v8bf, make_uint4(h0.x, h0.y, h1.x, h1.y));
    alo[cb] = __builtin_bit_cast(v8bf, make_uint4(l0.x, l0.y, l1.x, l1.y));
  }
  // B operands built once per pair and shared by the column blocks
  const uint64_t v01 = ((uint64_t)vsw[1] << 32) | vsw[0], v23 = ((uint64_t)vsw[3] << 32) | vsw[2];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    // words shifted in 64-bit pairs: bits crossing between the two words of a pair land
    // outside both masks (bits 3-6 and 19-22 of each word)
    const uint64_t s01 = q == 0 ? (v01 << 3) : (v01 >> (4 * q - 3));
    const uint64_t s23 = q == 0 ? (v23 << 3) : (v23 >> (4 * q - 3));
    const uint32_t y[4] = {(uint32_t)s01, (uint32_t)(s01 >> 32), (uint32_t)s23, (uint32_t)(s23 >> 32)};
    const v8bf ve = __builtin_bit_cast(v8bf, make_uint4(and_or(y[0], mask_e, magic), and_or(y[1], mask_e, magic),
                                                        and_or(y[2], mask_e, magic), and_or(y[3], mask_e, magic)));
    const v8bf vo = __builtin_bit_cast(v8bf, make_uint4(and_or(y[0], mask_o, magic), and_or(y[1], mask_o, magic),
                                                        and_or(y[2], mask_o, magic), and_or(y[3], mask_o, magic)));
    if constexpr (NCB == 8) {  // one accumulator set; the group's block supplies the rows
      const int bk = q >> 1;
      st.acc[0][2 * q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi[bk], ve, st.acc[0][2 * q], 0, 0, 0);
      st.acc[0][2 * q + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi[bk], vo, st.acc[0][2 * q + 1], 0, 0, 0);
      st.acc[0][2 * q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo[bk], ve, st.acc[0][2 * q], 0, 0, 0);
      st.acc[0][2 * q + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo[bk], vo, st.acc[0][2 * q + 1], 0, 0, 0);
      continue;
    }
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      st.acc[cb][2 * q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi[cb], ve, st.acc[cb][2 * q], 0, 0, 0);
      st.acc[cb][2 * q + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi[cb], vo, st.acc[cb][2 * q + 1], 0, 0, 0);
      st.acc[cb][2 * q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo[cb], ve, st.acc[cb][2 * q], 0, 0, 0);
      st.acc[cb][2 * q + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo[cb], vo, st.acc[cb][2 * q + 1], 0, 0, 0);
    }
  }
  // the same weights against a column of ones: the exact bf16 weight sums that the code
  // accumulators carry in their "1 +" part
#pragma unroll
  for (int cb = 0; cb < kLaneHeads<NCB>; ++cb) {
    st.wsum[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi[cb], ones, st.wsum[cb], 0, 0, 0);
    st.wsum[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo[cb], ones, st.wsum[cb], 0, 0, 0);
  }
}

// Priority of a worker wave after `band` quarters of its run (3 at the start, 0 in the last).
__device__ __forceinline__ void lower_priority(int band) {
  if (band == 1) __builtin_amdgcn_s_setprio(2);
  else if (band == 2) __builtin_amdgcn_s_setprio(1);
  else __builtin_amdgcn_s_setprio(0);
}

// Worker waves per workgroup: each wave is an independent worker with its own LDS ring and
// tile; two per workgroup lets a CU hold more than 16 workers.
constexpr int kWaves = 2;

// Shared memory of one workgroup of int2_decode_kernel: the page rings and W tiles of its
// INT2 workers, or the scratch of the BF16 window role.
template <int NCB>
constexpr size_t kSmemBytes = (size_t)kWaves * kRingBytes + (size_t)kWaves * sizeof(WTile<NCB>);

// BF16 sink + window positions of one (sequence, KV head), computed by the kWaves waves of one
// workgroup: logits on the bf16 MFMA (q' as a hi/lo bf16 pair, K rows exact), softmax in fp32,
// P.V on the VALU with one channel pair per lane.  With nparts > 1 the pair's positions (sink
// first, then window, in position order) are cut into parts of kWinPartTokens and this
// workgroup takes part `part`; with nparts == 1 it takes them all.  Written as window slot
// `part` of the pair; part 0 also marks window slots nparts .. kWinSlots-1 empty.
template <int NCB>
__device__ __forceinline__ void window_pair(const CacheGeom& g, const uint16_t* __restrict__ sinkwin,
                                            const int32_t* __restrict__ slot_ids, int hq,
                                            const int32_t* __restrict__ seq_lens, float sm_log2,
                                            const Workspace& ws, int b, int h, int part,
                                            int nparts, uint8_t* smem) {
  constexpr int kJ = 4 * NCB;  // head rows kept (G <= kJ)
  static_assert(kWaves == 2, "the P.V partials of the two waves are added pairwise");
  static_assert((kMaxSinkWindow * kJ + 2 * kJ + kJ * kHeadDim) * sizeof(float) <= kSmemBytes<NCB>,
                "window scratch exceeds the workgroup's shared memory");
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = hq / g.hkv;
  const int L = max(seq_lens[b], 0);
  const int slot = slot_ids ? slot_ids[b] : b;
  const int n_sink = min(L, g.num_sink);
  const int n_win = min(g.window, L - n_sink);
  const bool live = sinkwin != nullptr && slot >= 0 && slot < g.num_slots && n_sink + n_win > 0;
  const int n_all = live ? n_sink + n_win : 0;
  const int t0 = nparts == 1 ? 0 : part * kWinPartTokens;  // first position index of the part
  const int n = nparts == 1 ? n_all : min(max(n_all - t0, 0), kWinPartTokens);
  float* s_p = reinterpret_cast<float*>(smem);   // [kMaxSinkWindow][kJ] logits, then p
  float* s_red = s_p + kMaxSinkWindow * kJ;      // [kJ] max, then [kJ] sum
  float* s_o = s_red + 2 * kJ;                   // [kJ][128] P.V of the second wave
  const size_t base = ((size_t)slot * g.hkv + h) * (size_t)(g.num_sink + g.window);
  auto row_ptr = [&](int il) -> const uint16_t* {  // K row of part index il; the V row follows
    const int i = t0 + il;
    const int p = i < n_sink ? i : L - n_win + (i - n_sink);
    const int row = p < g.num_sink ? p : g.num_sink + p % g.window;
    return sinkwin + (base + row) * 2 * kHeadDim;
  };

  // Logits: S[j][token] = q'[j] . K[token], 16 tokens per tile.  A row m = lane % 16 is head m
  // (0 beyond G) holding channels 32*kq + 4*s .. +3 at step s (kq = lane / 16); the B column of
  // the same lane is token m of the tile with the same channels, read straight from its row.
  const int m = lane & 15, kq = lane >> 4;
  v4s qhi[8], qlo[8];
  {
    const float* qrow = reinterpret_cast<const float*>(ws.qblock(b, hq, h * G + (m < G ? m : 0)));
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      float4 v = *reinterpret_cast<const float4*>(qrow + 32 * kq + 4 * s);
      if (m >= G) v = make_float4(0.f, 0.f, 0.f, 0.f);
      const float w[4] = {v.x, v.y, v.z, v.w};
      uint32_t h01, h23, l01, l23;
      split_bf16(w, h01, h23, l01, l23);
      qhi[s] = __builtin_bit_cast(v4s, make_uint2(h01, h23));
      qlo[s] = __builtin_bit_cast(v4s, make_uint2(l01, l23));
    }
  }
  // Two tiles per wave per round, both tiles' K rows loaded before either is used.
  const int ntiles = (n + kPage - 1) / kPage;
  for (int tl0 = wave; tl0 < ntiles; tl0 += 2 * kWaves) {
    uint4 kr[2][4] = {};
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      const int i = (tl0 + h2 * kWaves) * kPage + m;
      if (i < n) {
        const uint4* kp = reinterpret_cast<const uint4*>(row_ptr(i) + 32 * kq);
#pragma unroll
        for (int u = 0; u < 4; ++u) kr[h2][u] = kp[u];
      }
    }
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      const int i = (tl0 + h2 * kWaves) * kPage + m;
      v4f d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const uint4& u = kr[h2][s >> 1];
        const v4s kb = __builtin_bit_cast(v4s, (s & 1) ? make_uint2(u.z, u.w) : make_uint2(u.x, u.y));
        d = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(qhi[s], kb, d, 0, 0, 0);
        d = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(qlo[s], kb, d, 0, 0, 0);
      }
      // D: this lane holds token i (column lane % 16) for heads 4*kq + e
      if (i < n) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (4 * kq + e < kJ) s_p[i * kJ + 4 * kq + e] = d[e] * sm_log2;
      }
    }
  }

  // P.V operands: lane -> channels 8*cq .. 8*cq + 7 (one 16-byte load) of token 4*k + tq of
  // the wave's token quads wave, wave + kWaves, ...; kVB loads per lane per round, the first
  // round issued before the softmax.
  const int cq = lane & 15, tq = lane >> 4;
  constexpr int kVB = 8;
  constexpr int kRound = 4 * kWaves * kVB;  // tokens per round of the workgroup
  auto load_v = [&](int i0, uint4 (&vv)[kVB]) {
#pragma unroll
    for (int u = 0; u < kVB; ++u) {
      const int i = i0 + 4 * kWaves * u + tq;
      vv[u] = i < n ? *reinterpret_cast<const uint4*>(row_ptr(i) + kHeadDim + 8 * cq)
                    : make_uint4(0u, 0u, 0u, 0u);
    }
  };
  uint4 vv[kVB];
  load_v(4 * wave, vv);
  __syncthreads();

  // Softmax per head over the n tokens: 16 threads per head.
  if (tid < kJ * 16) {
    const int j = tid >> 4, q = tid & 15;
    float mx = -INFINITY;
    for (int i = q; i < n; i += 16) mx = fmaxf(mx, s_p[i * kJ + j]);
    for (int o = 8; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
    float sum = 0.f;
    for (int i = q; i < n; i += 16) {
      const float p = __builtin_amdgcn_exp2f(s_p[i * kJ + j] - mx);
      s_p[i * kJ + j] = p;
      sum += p;
    }
    for (int o = 8; o >= 1; o >>= 1) sum += __shfl_xor(sum, o);
    if (q == 0) {
      s_red[j] = mx;
      s_red[kJ + j] = sum;
    }
  }
  __syncthreads();

  float acc[kJ][8];
#pragma unroll
  for (int j = 0; j < kJ; ++j)
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[j][c] = 0.f;
  for (int i0 = 4 * wave; i0 < n; i0 += kRound) {
    if (i0 > 4 * wave) load_v(i0, vv);
#pragma unroll
    for (int u = 0; u < kVB; ++u) {
      const int i = i0 + 4 * kWaves * u + tq;
      if (i < n) {
        const uint32_t w4[4] = {vv[u].x, vv[u].y, vv[u].z, vv[u].w};
#pragma unroll
        for (int j = 0; j < kJ; ++j) {
          const float p = s_p[i * kJ + j];
#pragma unroll
          for (int c2 = 0; c2 < 4; ++c2) {
            acc[j][2 * c2] = fmaf(p, __uint_as_float(w4[c2] << 16), acc[j][2 * c2]);
            acc[j][2 * c2 + 1] = fmaf(p, __uint_as_float(w4[c2] & 0xFFFF0000u), acc[j][2 * c2 + 1]);
          }
        }
      }
    }
  }
  // sum over the four token lanes of each channel group (fixed order), then over the waves
#pragma unroll
  for (int j = 0; j < kJ; ++j)
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      acc[j][c] += __shfl_xor(acc[j][c], 16);
      acc[j][c] += __shfl_xor(acc[j][c], 32);
    }
  if (wave == 1 && tq == 0) {
#pragma unroll
    for (int j = 0; j < kJ; ++j)
#pragma unroll
      for (int c = 0; c < 8; ++c) s_o[j * kHeadDim + 8 * cq + c] = acc[j][c];
  }
  __syncthreads();
  if (wave == 0) {
    const int out_slot = ws.win_slot() + part;
    if (part == 0) {  // the window slots no part of this launch writes
      for (int e = lane; e < G * (kWinSlots - nparts); e += 64)
        *ws.ml(b, hq, h * G + e % G, ws.win_slot() + nparts + e / G) = make_float2(kNegBig, 0.f);
    }
    if (tq == 0) {
#pragma unroll
      for (int j = 0; j < kJ; ++j)
        if (j < G) {
          float4* o = reinterpret_cast<float4*>(ws.o(b, hq, h * G + j, out_slot) + 8 * cq);
          const float* so = s_o + j * kHeadDim + 8 * cq;
          o[0] = make_float4(acc[j][0] + so[0], acc[j][1] + so[1], acc[j][2] + so[2], acc[j][3] + so[3]);
          o[1] = make_float4(acc[j][4] + so[4], acc[j][5] + so[5], acc[j][6] + so[6], acc[j][7] + so[7]);
        }
    }
    if (lane < G)
      *ws.ml(b, hq, h * G + lane, out_slot) =
          n > 0 ? make_float2(s_red[lane], s_red[kJ + lane]) : make_float2(kNegBig, 0.f);
  }
}


// NCB: the row layout (1 for G <= 4, 8 for G = 8; see kLaneHeads).
// worker_groups workgroups are INT2 workers, kWaves per workgroup.  Persistent part:
// worker w (one wavefront) takes run w of C pages of the concatenation of all (sequence, KV
// head) pairs' INT2 pages (the plan in the workspace, built by prep_q_kernel), and writes one
// partial for each pair its run touches, into that pair's slot w - (first run of the pair).
// Every worker therefore streams about the same number of pages.  batch * Hkv more workgroups
// compute the BF16 sink + window partial of one pair each: after the workers, so that they
// mostly run in the workers' tail, or (window_first, for launches with few pairs) before them.
template <int NCB>
__global__ __launch_bounds__(64 * kWaves) void int2_decode_kernel(
    CacheGeom g, const uint8_t* __restrict__ pages, const uint16_t* __restrict__ sinkwin,
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ slot_ids, int hq,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ plan, float sm_scale,
    int worker_groups, int window_first, int wparts, Workspace ws) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[kSmemBytes<NCB>];
  int bid = blockIdx.x;
  const int nwin = ws.batch * g.hkv * wparts;
  if (window_first ? bid < nwin : bid >= worker_groups) {
    const int widx = window_first ? bid : bid - worker_groups;
    const int pair = widx / wparts;
    window_pair<NCB == 8 ? 2 : NCB>(g, sinkwin, slot_ids, hq, seq_lens, sm_scale * kLog2e, ws,
                                    pair / g.hkv, pair % g.hkv, widx % wparts, wparts, smem);
    return;
  }
  if (window_first) bid -= nwin;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform per wavefront
  const int worker = bid * kWaves + wave;
  const int t = lane & 15, r = lane >> 4;
  WTile<NCB>& tile = *reinterpret_cast<WTile<NCB>*>(smem + (size_t)kWaves * kRingBytes +
                                                    wave * sizeof(WTile<NCB>));
  const uint32_t ring0 = lds_offset(smem + (size_t)wave * kRingBytes);
  // per-lane LDS offsets inside a pair slot (see read_pair_k / read_pair_v) and copy offset
  const uint32_t a8 = 8 * lane, a16 = 16 * t, voff = 16 * lane;
  const uint32_t vta = voff + 1024, vtb = voff + 512;  // tail copy offsets (see dma_pair)
  const uint32_t av = kPairHeadB * (r >> 1) + 512 + 256 * (r & 1) + 8 * t;

  const int total = plan[0], C = plan[1];
  if ((long long)worker * C >= total) return;
  // Equal-work waves on one SIMD would otherwise finish in dispatch order (the issue arbiter
  // prefers older waves) and leave the SIMD short of waves at the end; a wave lowers its
  // priority as it passes each quarter of its run, which lets the younger ones catch up.
  __builtin_amdgcn_s_setprio(3);
  const int band_len = max(C / 4, 1);
  int band_left = band_len, band = 0;
  const int run0 = worker * C;
  const int run1 = (int)min((long long)total, (long long)run0 + C);
  const int B = ws.batch;
  const int max_splits = ws.max_splits();
  const int32_t* pstart = plan + kPlanHeader;
  const int32_t* npg = pstart + B;
  const int32_t* pglo = npg + B;
  // sequence of the run's first page: the last b with pstart[b] <= run0 (it has pages).  The
  // wave probes 64 evenly spaced entries per round (pstart is non-decreasing, so the lanes that
  // pass form a prefix): one round for up to 64 sequences, two for up to 4096.
  int b = 0;
  {
    int len = B;   // the answer lies in [b, b + len); pstart[b] <= run0
    while (len > 1) {
      const int step = (len + 63) / 64;
      const bool probe = lane * step < len;
      const int v = pstart[probe ? b + lane * step : b];   // every index inside [b, b + len)
      const bool ok = probe && v <= run0;
      const int last = 63 - __clzll(__ballot(ok));   // lane 0 always passes
      b += last * step;
      len = min(step, len - last * step);
    }
  }
  const int G = hq / g.hkv;
  const float sm_log2 = sm_scale * kLog2e;
  const size_t rec_stride = (size_t)g.hkv * kRecord;  // bytes between pages of one head
  const uint32_t last_page = (uint32_t)(g.num_pages - 1);

  // Opaque copies of the V-code constants: masks in SGPRs, magic in a VGPR, so every
  // (x & mask) | magic is one instruction.  The empty asm statements emit nothing.
  uint32_t mask_e = 0x00180018u, mask_o = 0x00600060u, magic = 0x3F803F80u;
  asm volatile("" : "+s"(mask_e));
  asm volatile("" : "+s"(mask_o));
  asm volatile("" : "+v"(magic));
  const v8bf ones = __builtin_bit_cast(v8bf, make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u,
                                                        0x3F803F80u));  // bf16 1.0

  int pos = run0;
  while (true) {
    const int P = npg[b];
    const int rel = pos - pstart[b];
    const int h = rel / P;
    const int pair0 = pstart[b] + h * P;
    const int seg_end = min(run1, pair0 + P);
    const int slot = worker - pair0 / C;
    const int pgA = pglo[b] + (pos - pair0), pgB = pgA + (seg_end - pos);

    const int L = max(seq_lens[b], 0);
    const int n_sink = min(L, g.num_sink);
    const int lo = n_sink, hi = L - min(g.window, L - n_sink);

    QOperands<NCB> qo;
    if constexpr (NCB == 8) {
      // A-operand row of this lane: head t/2 with group t%2 (block 0, channel words 0..3) or
      // 2 + t%2 (block 1, words 4..7); quarter r holds word r of the block's half
      const char* blka = ws.qblock(b, hq, h * G + (t >> 1));
      const bool use = (r >> 1) == (t & 1);
      const v4i zero = {0, 0, 0, 0};
#pragma unroll
      for (int bk = 0; bk < 2; ++bk) {
        const v4i zh = *reinterpret_cast<const v4i*>(blka + kQHiOff + 16 * (4 * bk + r));
        const v4i zl = *reinterpret_cast<const v4i*>(blka + kQLoOff + 16 * (4 * bk + r));
        qo.hi[bk] = use ? zh : zero;
        qo.lo[bk] = use ? zl : zero;
      }
      // D rows of this lane: heads 2r and 2r + 1
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const char* blkd = ws.qblock(b, hq, h * G + 2 * r + hh);
        const float qsc = *reinterpret_cast<const float*>(blkd + kQScOff);
#pragma unroll
        for (int gg = 0; gg < 4; ++gg) qo.qs[hh][gg] = reinterpret_cast<const float*>(blkd + kQSumOff)[gg];
        qo.cscale[hh] = fmaxf(qsc / 254.0f * sm_log2, 1e-30f);
      }
    } else {
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
          qo.qs[cb][gg] = jd < G ? reinterpret_cast<const float*>(blkd + kQSumOff)[gg] : 0.f;
        // strictly positive so that a masked -inf logit never becomes 0 * inf
        qo.cscale[cb] = fmaxf(qsc / 254.0f * sm_log2, 1e-30f);
      }
    }

    const int32_t* bt = block_table + (size_t)b * g.max_pages;
    const uint8_t* pages_h = pages + (size_t)h * kRecord;  // record of (page 0, head h)
    SplitState<NCB> st;
#pragma unroll
    for (int cb = 0; cb < kLaneHeads<NCB>; ++cb) st.mref[cb] = kNegBig;
#pragma nounroll
    for (int pass = 0; pass < 2; ++pass) {
      const bool fixed_ref = pass > 0;
#pragma unroll
      for (int cs = 0; cs < kAccSets<NCB>; ++cs)
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) st.acc[cs][nb] = (v4f){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int cb = 0; cb < kLaneHeads<NCB>; ++cb) {
        st.lsum[cb] = 0.f;
        st.mlane[cb] = -INFINITY;
#pragma unroll
        for (int gg = 0; gg < 4; ++gg) st.zp[cb][gg] = 0.f;
        st.wsum[cb] = (v4f){0.f, 0.f, 0.f, 0.f};
      }

      // Page ids come from uniform (scalar) loads, fetched one page before they are used;
      // scalar loads are counted by lgkmcnt, so waiting for one never drains the page ring.
      // Each page issues exactly one record copy, so the per-page wait counts are exact.  An
      // id outside the pool reads page 0 instead (memory safety; the caller's table is wrong).
      // Pages in pairs [pgA + 2k, pgA + 2k + 1); a second page at or beyond pgB is a dummy
      // (it copies the segment's last page again and is masked).  An id outside the pool reads
      // the pool's last page instead (memory safety; the caller's table is wrong).  Page ids
      // come from uniform (scalar) loads, fetched one pair before they are used.
      const int npairs = (pgB - pgA + 1) >> 1;
      auto pslot = [&](int k) { return ring0 + (uint32_t)(k & 1) * kPairBytes; };
      int nidA = bt[pgA], nidB = bt[min(pgA + 1, pgB - 1)];  // ids of the next pair to issue
      int pfA = 0, pfB = 0;                                 // prefetched ids of the one after
      auto rec_of = [&](int id) {
        return pages_h + (size_t)min((uint32_t)id, last_page) * rec_stride;
      };
      auto issue = [&](int k) {  // issue pair k (its ids are in nidA / nidB)
        dma_pair(rec_of(nidA), rec_of(nidB), pslot(k), voff, vta, vtb);
      };
      auto prefetch = [&](int k) {  // ids of pair k
        const int pg = pgA + 2 * k;
        pfA = bt[min(pg, pgB - 1)];
        pfB = bt[min(pg + 1, pgB - 1)];
      };
      auto band_tick = [&]() {
        band_left -= 2;
        if (__builtin_expect(band_left <= 0, 0)) {
          band_left += band_len;
          lower_priority(++band);
        }
      };
      auto live_at = [&](int q) {
        const int p = q * kPage + t;
        return q < pgB && p >= lo && p < hi;
      };

      issue(0);
      if (npairs > 1) {  // pair 1 is issued before pair 0 is waited for
        prefetch(1);
        nidA = pfA;
        nidB = pfB;
        issue(1);
        prefetch(2);
        wait_pairs<1>();
      } else {
        wait_pairs<0>();
      }
      // first pair (page A may hold sink positions; both pages may hold window positions or
      // the end when it is also the last pair)
      int2_pair<NCB, true, true>(pslot(0), a8, a16, av, live_at(pgA), live_at(pgA + 1), qo, st,
                                 tile, t, r, mask_e, mask_o, magic, ones, fixed_ref, [] {});
      int k = 1;
      for (; k < npairs - 1; ++k) {  // interior pairs: every position is INT2
        band_tick();
        nidA = pfA;
        nidB = pfB;
        issue(k + 1);
        wait_pairs<1>();
        int2_pair<NCB, false, false>(pslot(k), a8, a16, av, true, true, qo, st, tile, t, r,
                                     mask_e, mask_o, magic, ones, fixed_ref,
                                     [&] { prefetch(k + 2); });
      }
      if (k == npairs - 1) {  // last pair (k >= 1)
        wait_pairs<0>();
        const int pg = pgA + 2 * k;
        int2_pair<NCB, true, false>(pslot(k), a8, a16, av, live_at(pg), live_at(pg + 1), qo, st,
                                    tile, t, r, mask_e, mask_o, magic, ones, fixed_ref, [] {});
      }

      // A logit beyond the reference margin: recompute once with the exact max (rare path).
      bool redo = false;
      float mexact[kLaneHeads<NCB>];
#pragma unroll
      for (int cb = 0; cb < kLaneHeads<NCB>; ++cb) {
        mexact[cb] = row_max16(st.mlane[cb]) * qo.cscale[cb];
        redo |= mexact[cb] > st.mref[cb] + kRefMargin;
      }
      if (pass > 0 || !__any(redo)) break;
#pragma unroll
      for (int cb = 0; cb < kLaneHeads<NCB>; ++cb) st.mref[cb] = mexact[cb];
    }

    // Finish: l and the per-group sums reduced over the row's 16 tokens; the accumulator row
    // of a lane (head 4*cb + r) matches its own row, so no exchange is needed.
    //   o'[c] = sum_t p_t (s_t code_t(c) + z_t) = f (acc - sum_t W_t) + sum_t p_t z_t
    // with f = 16 or 4 for the block's code scale and W_t the bf16 weight pair.
    if constexpr (NCB == 8) {
      // lane head hh = head 2r + hh; its row in block g/2 for group g is element 2hh + g%2
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const float lt = row_sum16(st.lsum[hh]);
        float zt[4];
#pragma unroll
        for (int gg = 0; gg < 4; ++gg) zt[gg] = row_sum16(st.zp[hh][gg]);
        const int j = 2 * r + hh;
        if ((unsigned)slot < (unsigned)max_splits) {
          float* o = ws.o(b, hq, h * G + j, slot);
#pragma unroll
          for (int nb = 0; nb < 8; ++nb) {
            const int gg = nb >> 1, i = 2 * hh + (gg & 1);
            o[16 * nb + t] = fmaf(kVScale[nb & 1], st.acc[0][nb][i] - st.wsum[gg >> 1][i], zt[gg]);
          }
          if (t == 0) *ws.ml(b, hq, h * G + j, slot) = make_float2(st.mref[hh], lt);
        }
      }
    } else {
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      const float lt = row_sum16(st.lsum[cb]);
      float zt[4], wt[4];
#pragma unroll
      for (int gg = 0; gg < 4; ++gg) {
        zt[gg] = row_sum16(st.zp[cb][gg]);
        wt[gg] = st.wsum[cb][gg];
      }
      const int j = 4 * cb + r;
      if (j < G && (unsigned)slot < (unsigned)max_splits) {
        float* o = ws.o(b, hq, h * G + j, slot);
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) {
          const int gg = nb >> 1;
          o[16 * nb + t] = fmaf(kVScale[nb & 1], st.acc[cb][nb][gg] - wt[gg], zt[gg]);
        }
        if (t == 0) *ws.ml(b, hq, h * G + j, slot) = make_float2(st.mref[cb], lt);
      }
    }
    }

    pos = seg_end;
    if (pos >= run1) break;
    if (h == g.hkv - 1) {
      do { ++b; } while (b < B - 1 && npg[b] == 0);
    }
  }
}

// ------------------------------------------------------------------ INT4 pages, matrix cores
//
// The INT4 variant's decode for G <= 4 (the INT4 abstract on the OSCAR paper's page: token-wise
// INT4 through the same paged path).  The same workers, plan, q' encoding, sink/window role and
// partial format as int2_decode_kernel<1>; what changes is the page: 2560-byte records copied
// one page at a time into a two-page LDS ring (three direct-to-LDS loads per page, the next page
// in flight while one is computed), K codes read as int8 operands with two nibble masks (the
// record keeps the INT2 operand order, so q' is encoded once for both), and P.V per page on
// v_mfma_f32_16x16x16_bf16 with V codes as bf16 1 + code/16 built from one shift and one AND-OR
// per two tokens (every column block scales by 16).

constexpr int kPage4Bytes = 2560;
constexpr int kRing4Bytes = 2 * kPage4Bytes;
template <int NCB>
constexpr size_t kSmem4Bytes = (size_t)kWaves * kRing4Bytes + (size_t)kWaves * sizeof(WTile<NCB>);
static_assert((kMaxSinkWindow * 4 + 2 * 4 + 4 * kHeadDim) * sizeof(float) <= kSmem4Bytes<1> &&
                  (kMaxSinkWindow * 8 + 2 * 8 + 8 * kHeadDim) * sizeof(float) <= kSmem4Bytes<8>,
              "window scratch exceeds the INT4 workgroup's shared memory");

// Copy the record at rec (uniform) into the page slot at LDS offset ps: bytes [0, 1024) and
// [1024, 2048) by full-wave loads, [2048, 2560) by lanes 0..31 (exec restricted inside the
// statement and restored before it ends).  Lane l's 16 bytes land at M0 + 16 l; v0 = 16 l.
__device__ __forceinline__ void dma_page4(const uint8_t* rec, uint32_t ps, uint32_t v0) {
  uint64_t saved;
  const uint32_t ps1 = __builtin_amdgcn_readfirstlane(ps + 0x400u);
  const uint32_t ps2 = __builtin_amdgcn_readfirstlane(ps + 0x800u);
  asm volatile(
      "s_mov_b32 m0, %[ps]\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %[v0], %[a]\n\t"
      "s_mov_b32 m0, %[ps1]\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %[v1], %[a]\n\t"
      "s_mov_b32 m0, %[ps2]\n\t"
      "s_mov_b64 %[sv], exec\n\t"
      "s_mov_b32 exec_hi, 0\n\t"
      "global_load_lds_dwordx4 %[v2], %[a]\n\t"
      "s_mov_b64 exec, %[sv]"
      : [sv] "=&s"(saved)
      : [ps] "s"(ps), [ps1] "s"(ps1), [ps2] "s"(ps2), [v0] "v"(v0), [v1] "v"(v0 + 1024u),
        [v2] "v"(v0 + 2048u), [a] "s"(rec)
      : "memory", "m0");
}

// Wait until at most N pages' copies (3 loads each) are still outstanding.
template <int N>
__device__ __forceinline__ void wait_pages4() {
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(3 * N) : "memory");
}

// This lane's view of a page slot: its K chunk (quarter r, token t) and the K (scale, zero) of
// token t; then the V (scale, zero) of token t and its V chunk (token quad r, channel residue
// t).  a16l = 16 lane, a16t = 16 t.
__device__ __forceinline__ void read_page4_k(uint32_t ps, uint32_t a16l, uint32_t a16t,
                                             uint4& kc, uint4& km) {
  asm volatile(
      "ds_read_b128 %0, %2\n\t"
      "ds_read_b128 %1, %3 offset:2048\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(kc), "=&v"(km)
      : "v"(ps + a16l), "v"(ps + a16t)
      : "memory");
}
__device__ __forceinline__ void read_page4_v(uint32_t ps, uint32_t a16l, uint32_t a16t,
                                             uint4& vm, uint4& vc) {
  asm volatile(
      "ds_read_b128 %0, %3 offset:2304\n\t"
      "ds_read_b128 %1, %2 offset:1024\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(vm), "=&v"(vc)
      : "v"(ps + a16l), "v"(ps + a16t)
      : "memory");
}

// Logit of head r, token t in units of cscale (as page_logits<1>): the chunk's dwords masked
// with 0x0F0F0F0F at shifts 0 and 4 are the two int8 K operands.
template <int NCB, bool MASKED>
__device__ __forceinline__ void page4_logits(uint4 kc, uint4 km, bool live, const QOperands<NCB>& qo,
                                             uint32_t m4, float a[kLaneHeads<NCB>]) {
  const v4i ka0 = (v4i){(int)(kc.x & m4), (int)((kc.x >> 4) & m4), (int)(kc.y & m4),
                        (int)((kc.y >> 4) & m4)};
  const v4i ka1 = (v4i){(int)(kc.z & m4), (int)((kc.z >> 4) & m4), (int)(kc.w & m4),
                        (int)((kc.w >> 4) & m4)};
  const uint32_t kmw[4] = {km.x, km.y, km.z, km.w};
  // |dh| <= 127 * 15 * 32 per group: 254 dh + dl stays below 2^24, exact in fp32
  if constexpr (NCB == 8) {
    // the INT2 G = 8 row layout: D element i of a lane is head 2r + i/2, group i%2 (block A,
    // channels 0..63) or 2 + i%2 (block B, channels 64..127)
    const v4i zero = {0, 0, 0, 0};
    const v4i dhA = __builtin_amdgcn_mfma_i32_16x16x64_i8(qo.hi[0], ka0, zero, 0, 0, 0);
    const v4i dlA = __builtin_amdgcn_mfma_i32_16x16x64_i8(qo.lo[0], ka0, zero, 0, 0, 0);
    const v4i dhB = __builtin_amdgcn_mfma_i32_16x16x64_i8(qo.hi[1], ka1, zero, 0, 0, 0);
    const v4i dlB = __builtin_amdgcn_mfma_i32_16x16x64_i8(qo.lo[1], ka1, zero, 0, 0, 0);
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      float x = 0.f;
#pragma unroll
      for (int gl = 0; gl < 2; ++gl) {
        const int i = 2 * hh + gl;
        const int dA = __mul24(dhA[i], 254) + dlA[i], dB = __mul24(dhB[i], 254) + dlB[i];
        x = fmaf(f16lo(kmw[gl]), (float)dA, x);
        x = fmaf(f16hi(kmw[gl]), qo.qs[hh][gl], x);
        x = fmaf(f16lo(kmw[2 + gl]), (float)dB, x);
        x = fmaf(f16hi(kmw[2 + gl]), qo.qs[hh][2 + gl], x);
      }
      if (MASKED) x = live ? x : -INFINITY;
      a[hh] = x;
    }
  } else {
    v4i dh = {0, 0, 0, 0}, dl = {0, 0, 0, 0};
    dh = __builtin_amdgcn_mfma_i32_16x16x64_i8(qo.hi[0][0], ka0, dh, 0, 0, 0);
    dh = __builtin_amdgcn_mfma_i32_16x16x64_i8(qo.hi[0][1], ka1, dh, 0, 0, 0);
    dl = __builtin_amdgcn_mfma_i32_16x16x64_i8(qo.lo[0][0], ka0, dl, 0, 0, 0);
    dl = __builtin_amdgcn_mfma_i32_16x16x64_i8(qo.lo[0][1], ka1, dl, 0, 0, 0);
    float x = 0.f;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int dint = __mul24(dh[g], 254) + dl[g];
      x = fmaf(f16lo(kmw[g]), (float)dint, x);
      x = fmaf(f16hi(kmw[g]), qo.qs[0][g], x);
    }
    if (MASKED) x = live ? x : -INFINITY;
    a[0] = x;
  }
}

// One page in the slot at ps: logits, weights into the tile (columns 0..15), P.V and the weight
// sums.  after_reads() runs once the slot's LDS reads have completed (the copy of a later page
// into the slot goes there).
template <int NCB, bool MASKED, bool FIRST, class AfterReads>
__device__ __forceinline__ void int4_page(uint32_t ps, uint32_t a16l, uint32_t a16t, bool live,
                                          const QOperands<NCB>& qo, SplitState<NCB>& st,
                                          WTile<NCB>& tile, int t, int r, uint32_t m4,
                                          uint32_t mask_v, uint32_t magic, v4s ones,
                                          bool fixed_ref, AfterReads&& after_reads) {
  uint4 kc, km;
  read_page4_k(ps, a16l, a16t, kc, km);
  float a[kLaneHeads<NCB>];
  page4_logits<NCB, MASKED>(kc, km, live, qo, m4, a);
#pragma unroll
  for (int cb = 0; cb < kLaneHeads<NCB>; ++cb) {
    st.mlane[cb] = fmaxf(st.mlane[cb], a[cb]);
    if (FIRST && !fixed_ref) st.mref[cb] = fmaxf(row_max16(a[cb]) * qo.cscale[cb], kNegBig);
  }
  uint4 vm, vc;
  read_page4_v(ps, a16l, a16t, vm, vc);
  after_reads();
  page_weights<NCB, MASKED>(a, vm, live, qo, st, tile, t, r, 0);
  // A operands of each row block: row t of the tile, tokens 4r .. 4r + 3
  v4s ahi[kLaneHeads<NCB>], alo[kLaneHeads<NCB>];
#pragma unroll
  for (int cb = 0; cb < kLaneHeads<NCB>; ++cb) {
    const uint2 h2 = *reinterpret_cast<const uint2*>(&tile.w[cb][0][t][4 * r]);
    const uint2 l2 = *reinterpret_cast<const uint2*>(&tile.w[cb][1][t][4 * r]);
    ahi[cb] = __builtin_bit_cast(v4s, h2);
    alo[cb] = __builtin_bit_cast(v4s, l2);
  }
  const uint32_t vw[4] = {vc.x, vc.y, vc.z, vc.w};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t w = vw[k];
    // column block 2k: tokens (0, 1) from w << 3, (2, 3) from w >> 5; block 2k + 1: w >> 1, w >> 9
    const v4s b0 = __builtin_bit_cast(v4s, make_uint2(and_or(w << 3, mask_v, magic),
                                                      and_or(w >> 5, mask_v, magic)));
    const v4s b1 = __builtin_bit_cast(v4s, make_uint2(and_or(w >> 1, mask_v, magic),
                                                      and_or(w >> 9, mask_v, magic)));
    // column blocks 2k, 2k + 1 are group k: G = 8 takes the row block of its group pair
    const int bk = NCB == 8 ? (k >> 1) : 0;
    st.acc[0][2 * k] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ahi[bk], b0, st.acc[0][2 * k], 0, 0, 0);
    st.acc[0][2 * k] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(alo[bk], b0, st.acc[0][2 * k], 0, 0, 0);
    st.acc[0][2 * k + 1] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ahi[bk], b1, st.acc[0][2 * k + 1], 0, 0, 0);
    st.acc[0][2 * k + 1] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(alo[bk], b1, st.acc[0][2 * k + 1], 0, 0, 0);
  }
#pragma unroll
  for (int cb = 0; cb < kLaneHeads<NCB>; ++cb) {
    st.wsum[cb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ahi[cb], ones, st.wsum[cb], 0, 0, 0);
    st.wsum[cb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(alo[cb], ones, st.wsum[cb], 0, 0, 0);
  }
}

// grid: worker_groups INT2-style worker workgroups (kWaves workers each) and batch * Hkv *
// wparts sink/window workgroups, ordered as in int2_decode_kernel.  NCB: the row layout of
// int2_decode_kernel (1 for G <= 4, 8 for G = 8).
template <int NCB>
__global__ __launch_bounds__(64 * kWaves) __attribute__((amdgpu_waves_per_eu(3))) void int4_decode_mfma_kernel(
    CacheGeom g, const uint8_t* __restrict__ pages, const uint16_t* __restrict__ sinkwin,
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ slot_ids, int hq,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ plan, float sm_scale,
    int worker_groups, int window_first, int wparts, Workspace ws) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[kSmem4Bytes<NCB>];
  int bid = blockIdx.x;
  const int nwin = ws.batch * g.hkv * wparts;
  if (window_first ? bid < nwin : bid >= worker_groups) {
    const int widx = window_first ? bid : bid - worker_groups;
    const int pair = widx / wparts;
    window_pair<NCB == 8 ? 2 : NCB>(g, sinkwin, slot_ids, hq, seq_lens, sm_scale * kLog2e, ws,
                                    pair / g.hkv, pair % g.hkv, widx % wparts, wparts, smem);
    return;
  }
  if (window_first) bid -= nwin;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int worker = bid * kWaves + wave;
  const int t = lane & 15, r = lane >> 4;
  WTile<NCB>& tile = *reinterpret_cast<WTile<NCB>*>(smem + (size_t)kWaves * kRing4Bytes +
                                                    wave * sizeof(WTile<NCB>));
  const uint32_t ring0 = lds_offset(smem + (size_t)wave * kRing4Bytes);
  const uint32_t a16l = 16 * lane, a16t = 16 * t;

  const int total = plan[0], C = plan[1];
  if ((long long)worker * C >= total) return;
  __builtin_amdgcn_s_setprio(3);
  const int band_len = max(C / 4, 1);
  int band_left = band_len, band = 0;
  const int run0 = worker * C;
  const int run1 = (int)min((long long)total, (long long)run0 + C);
  const int B = ws.batch;
  const int max_splits = ws.max_splits();
  const int32_t* pstart = plan + kPlanHeader;
  const int32_t* npg = pstart + B;
  const int32_t* pglo = npg + B;
  int b = 0;
  {
    int len = B;
    while (len > 1) {
      const int step = (len + 63) / 64;
      const bool probe = lane * step < len;
      const int v = pstart[probe ? b + lane * step : b];
      const bool ok = probe && v <= run0;
      const int last = 63 - __clzll(__ballot(ok));
      b += last * step;
      len = min(step, len - last * step);
    }
  }
  const int G = hq / g.hkv;
  const float sm_log2 = sm_scale * kLog2e;
  const size_t rec_stride = (size_t)g.hkv * kPage4Bytes;
  const uint32_t last_page = (uint32_t)(g.num_pages - 1);
  uint32_t m4 = 0x0F0F0F0Fu, mask_v = 0x00780078u, magic = 0x3F803F80u;
  asm volatile("" : "+s"(m4));
  asm volatile("" : "+s"(mask_v));
  asm volatile("" : "+v"(magic));
  const v4s ones = __builtin_bit_cast(v4s, make_uint2(0x3F803F80u, 0x3F803F80u));  // bf16 1.0

  int pos = run0;
  while (true) {
    const int P = npg[b];
    const int rel = pos - pstart[b];
    const int h = rel / P;
    const int pair0 = pstart[b] + h * P;
    const int seg_end = min(run1, pair0 + P);
    const int slot = worker - pair0 / C;
    const int pgA = pglo[b] + (pos - pair0), pgB = pgA + (seg_end - pos);

    const int L = max(seq_lens[b], 0);
    const int n_sink = min(L, g.num_sink);
    const int lo = n_sink, hi = L - min(g.window, L - n_sink);

    QOperands<NCB> qo;
    if constexpr (NCB == 8) {
      // A-operand row of this lane: head t/2 with group t%2 (block 0, channel words 0..3) or
      // 2 + t%2 (block 1, words 4..7); quarter r holds word r of the block's half
      const char* blka = ws.qblock(b, hq, h * G + (t >> 1));
      const bool use = (r >> 1) == (t & 1);
      const v4i zero = {0, 0, 0, 0};
#pragma unroll
      for (int bk = 0; bk < 2; ++bk) {
        const v4i zh = *reinterpret_cast<const v4i*>(blka + kQHiOff + 16 * (4 * bk + r));
        const v4i zl = *reinterpret_cast<const v4i*>(blka + kQLoOff + 16 * (4 * bk + r));
        qo.hi[bk] = use ? zh : zero;
        qo.lo[bk] = use ? zl : zero;
      }
      // D rows of this lane: heads 2r and 2r + 1
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const char* blkd = ws.qblock(b, hq, h * G + 2 * r + hh);
        const float qsc = *reinterpret_cast<const float*>(blkd + kQScOff);
#pragma unroll
        for (int gg = 0; gg < 4; ++gg) qo.qs[hh][gg] = reinterpret_cast<const float*>(blkd + kQSumOff)[gg];
        qo.cscale[hh] = fmaxf(qsc / 254.0f * sm_log2, 1e-30f);
      }
    } else {
      const int ja = t >> 2, ga = t & 3;
      const char* blka = ws.qblock(b, hq, h * G + (ja < G ? ja : 0));
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const int dw = 4 * m + r;
        const bool use = ja < G && (dw >> 1) == ga;
        const v4i zh = *reinterpret_cast<const v4i*>(blka + kQHiOff + 16 * dw);
        const v4i zl = *reinterpret_cast<const v4i*>(blka + kQLoOff + 16 * dw);
        const v4i zero = {0, 0, 0, 0};
        qo.hi[0][m] = use ? zh : zero;
        qo.lo[0][m] = use ? zl : zero;
      }
      const int jd = r;
      const char* blkd = ws.qblock(b, hq, h * G + (jd < G ? jd : 0));
      const float qsc = jd < G ? *reinterpret_cast<const float*>(blkd + kQScOff) : 0.f;
#pragma unroll
      for (int gg = 0; gg < 4; ++gg)
        qo.qs[0][gg] = jd < G ? reinterpret_cast<const float*>(blkd + kQSumOff)[gg] : 0.f;
      qo.cscale[0] = fmaxf(qsc / 254.0f * sm_log2, 1e-30f);
    }

    const int32_t* bt = block_table + (size_t)b * g.max_pages;
    const uint8_t* pages_h = pages + (size_t)h * kPage4Bytes;
    SplitState<NCB> st;
#pragma unroll
    for (int cb = 0; cb < kLaneHeads<NCB>; ++cb) st.mref[cb] = kNegBig;
#pragma nounroll
    for (int pass = 0; pass < 2; ++pass) {
      const bool fixed_ref = pass > 0;
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) st.acc[0][nb] = (v4f){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int cb = 0; cb < kLaneHeads<NCB>; ++cb) {
        st.lsum[cb] = 0.f;
        st.mlane[cb] = -INFINITY;
#pragma unroll
        for (int gg = 0; gg < 4; ++gg) st.zp[cb][gg] = 0.f;
        st.wsum[cb] = (v4f){0.f, 0.f, 0.f, 0.f};
      }

      // Pages pgA .. pgB-1, two in flight; page ids from uniform (scalar) loads one page ahead
      // of their copy.  An id outside the pool reads the pool's last page (memory safety).
      const int np = pgB - pgA;
      auto pslot = [&](int k) { return ring0 + (uint32_t)(k & 1) * kPage4Bytes; };
      auto rec_of = [&](int id) {
        return pages_h + (size_t)min((uint32_t)id, last_page) * rec_stride;
      };
      auto live_at = [&](int q) {
        const int p = q * kPage + t;
        return q < pgB && p >= lo && p < hi;
      };
      int pf = bt[pgA];
      dma_page4(rec_of(pf), pslot(0), a16l);
      if (np > 1) {
        pf = bt[pgA + 1];
        dma_page4(rec_of(pf), pslot(1), a16l);
      }
      pf = np > 2 ? bt[pgA + 2] : 0;
      for (int k = 0; k < np; ++k) {
        if (k + 1 < np) wait_pages4<1>();
        else wait_pages4<0>();
        auto next = [&] {  // the slot just read takes page k + 2
          if (k + 2 < np) {
            dma_page4(rec_of(pf), pslot(k), a16l);
            pf = k + 3 < np ? bt[pgA + k + 3] : 0;
          }
        };
        if (--band_left <= 0) {
          band_left += band_len;
          lower_priority(++band);
        }
        const int q = pgA + k;
        if (k == 0)
          int4_page<NCB, true, true>(pslot(k), a16l, a16t, live_at(q), qo, st, tile, t, r, m4,
                                     mask_v, magic, ones, fixed_ref, next);
        else if (k == np - 1)
          int4_page<NCB, true, false>(pslot(k), a16l, a16t, live_at(q), qo, st, tile, t, r, m4,
                                      mask_v, magic, ones, fixed_ref, next);
        else
          int4_page<NCB, false, false>(pslot(k), a16l, a16t, true, qo, st, tile, t, r, m4, mask_v,
                                       magic, ones, fixed_ref, next);
      }

      // A logit beyond the reference margin: recompute once with the exact max (rare path).
      bool redo = false;
      float mexact[kLaneHeads<NCB>];
#pragma unroll
      for (int cb = 0; cb < kLaneHeads<NCB>; ++cb) {
        mexact[cb] = row_max16(st.mlane[cb]) * qo.cscale[cb];
        redo |= mexact[cb] > st.mref[cb] + kRefMargin;
      }
      if (pass > 0 || !__any(redo)) break;
#pragma unroll
      for (int cb = 0; cb < kLaneHeads<NCB>; ++cb) st.mref[cb] = mexact[cb];
    }

    // Finish (as int2_decode_kernel<NCB>): o'[c] = 16 (acc - sum_t W_t) + sum_t p_t z_t.
    if constexpr (NCB == 8) {
      // lane head hh = head 2r + hh; its row in block g/2 for group g is element 2hh + g%2
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const float lt = row_sum16(st.lsum[hh]);
        float zt[4];
#pragma unroll
        for (int gg = 0; gg < 4; ++gg) zt[gg] = row_sum16(st.zp[hh][gg]);
        const int j = 2 * r + hh;
        if ((unsigned)slot < (unsigned)max_splits) {
          float* o = ws.o(b, hq, h * G + j, slot);
#pragma unroll
          for (int nb = 0; nb < 8; ++nb) {
            const int gg = nb >> 1, i = 2 * hh + (gg & 1);
            o[16 * nb + t] = fmaf(16.0f, st.acc[0][nb][i] - st.wsum[gg >> 1][i], zt[gg]);
          }
          if (t == 0) *ws.ml(b, hq, h * G + j, slot) = make_float2(st.mref[hh], lt);
        }
      }
    } else {
      const float lt = row_sum16(st.lsum[0]);
      float zt[4];
#pragma unroll
      for (int gg = 0; gg < 4; ++gg) zt[gg] = row_sum16(st.zp[0][gg]);
      const int j = r;
      if (j < G && (unsigned)slot < (unsigned)max_splits) {
        float* o = ws.o(b, hq, h * G + j, slot);
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) {
          const int gg = nb >> 1;
          o[16 * nb + t] = fmaf(16.0f, st.acc[0][nb][gg] - st.wsum[0][gg], zt[gg]);
        }
        if (t == 0) *ws.ml(b, hq, h * G + j, slot) = make_float2(st.mref[0], lt);
      }
    }

    pos = seg_end;
    if (pos >= run1) break;
    if (h == g.hkv - 1) {
      do { ++b; } while (b < B - 1 && npg[b] == 0);
    }
  }
}

// Resident worker waves of int2_decode_kernel<NCB> on the current device (cached per device).
template <int NCB>
int resident_workers() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cache[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) dev = 0;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n > 0) return n;
  const int cus = current_device_cus();
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void*)int2_decode_kernel<NCB>,
                                                   64 * kWaves, 0) != hipSuccess)
    per_cu = 0;
  n = max(cus, 1) * max(per_cu, 1) * kWaves;
  cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

// Resident worker waves of int4_decode_mfma_kernel<NCB> on the current device (cached per device).
template <int NCB>
int int4_resident_workers() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cache[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) dev = 0;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n > 0) return n;
  const int cus = current_device_cus();
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void*)int4_decode_mfma_kernel<NCB>,
                                                   64 * kWaves, 0) != hipSuccess)
    per_cu = 0;
  n = max(cus, 1) * max(per_cu, 1) * kWaves;
  cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

}  // namespace

hipError_t launch_prep_q(const CacheGeom& g, const uint16_t* q, const float* rot_k, int batch,
                         int hq, const int32_t* seq_lens, const Workspace& ws, hipStream_t stream) {
  if (batch == 0) return hipSuccess;
  return launch_prep_q_grid(dim3(g.hkv, batch + 1), stream, g, q, rot_k, hq, seq_lens, 1,
                            hq / g.hkv, ws);
}

namespace {

// Launch shape of the INT2 decode (shared by its q preparation and the decode kernel, which must
// agree on the worker count the plan is built for).
struct DecodeShape {
  int G, workers, worker_groups, window_first, wparts, hpw;
};

DecodeShape decode_shape(const CacheGeom& g, int batch, int hq, int num_workers) {
  DecodeShape s;
  s.G = hq / g.hkv;
  s.workers = num_workers > 0 ? num_workers
                              : (s.G <= 4 ? resident_workers<1>() : resident_workers<8>());
  // Few pairs: their sink/window workgroups go first, so that they start at once instead of
  // after the INT2 workers that fill the device, each pair's positions are cut into parts of
  // kWinPartTokens (one workgroup each: a part's loads all go out in one round, where a whole
  // window takes several dependent rounds), and the q rotation takes one workgroup per query
  // head.  Many pairs: one window workgroup per pair, in the workers' tail.
  const int cus = current_device_cus();
  const bool small = (long long)batch * g.hkv * 2 < cus;
  s.window_first = small ? 1 : 0;
  s.wparts =
      small ? max(1, min(kWinSlots, (g.num_sink + g.window + kWinPartTokens - 1) / kWinPartTokens))
            : 1;
  s.hpw = small ? 1 : s.G;
  s.worker_groups = (s.workers + kWaves - 1) / kWaves;
  return s;
}

}  // namespace

hipError_t launch_decode_prep(const CacheGeom& g, const uint16_t* q, const float* rot_k, int batch,
                              int hq, const int32_t* seq_lens, int num_workers,
                              const Workspace& ws, hipStream_t stream) {
  if (batch == 0) return hipSuccess;
  const DecodeShape s = decode_shape(g, batch, hq, num_workers);
  return launch_prep_q_grid(dim3(g.hkv * (s.G / s.hpw), batch + 1), stream, g, q, rot_k, hq,
                            seq_lens, s.workers, s.hpw, ws);
}

void decode_prep_config(const CacheGeom& g, int batch, int hq, int num_workers, int* workers,
                        int* hpw) {
  const DecodeShape s = decode_shape(g, batch, hq, num_workers);
  *workers = s.workers;
  *hpw = s.hpw;
}

hipError_t launch_decode_main(const CacheGeom& g, const uint8_t* pages, const uint16_t* sinkwin,
                              const int32_t* block_table, const int32_t* slot_ids, int batch,
                              int hq, const int32_t* seq_lens, float sm_scale, int num_workers,
                              const Workspace& ws, hipStream_t stream) {
  if (batch == 0) return hipSuccess;
  const DecodeShape s = decode_shape(g, batch, hq, num_workers);
  const dim3 grid(s.worker_groups + batch * g.hkv * s.wparts);
  const int32_t* plan = ws.plan();
  if (s.G <= 4)
    hipLaunchKernelGGL(int2_decode_kernel<1>, grid, dim3(64 * kWaves), 0, stream, g, pages,
                       sinkwin, block_table, slot_ids, hq, seq_lens, plan, sm_scale,
                       s.worker_groups, s.window_first, s.wparts, ws);
  else
    hipLaunchKernelGGL(int2_decode_kernel<8>, grid, dim3(64 * kWaves), 0, stream, g, pages,
                       sinkwin, block_table, slot_ids, hq, seq_lens, plan, sm_scale,
                       s.worker_groups, s.window_first, s.wparts, ws);
  return hipGetLastError();
}

hipError_t launch_decode(const CacheGeom& g, const uint8_t* pages, const uint16_t* sinkwin,
                         const int32_t* block_table, const int32_t* slot_ids, int batch,
                         int hq, const uint16_t* q, const int32_t* seq_lens, const float* rot_k,
                         float sm_scale, int num_workers, const Workspace& ws,
                         hipStream_t stream) {
  const hipError_t e = launch_decode_prep(g, q, rot_k, batch, hq, seq_lens, num_workers, ws, stream);
  if (e != hipSuccess) return e;
  return launch_decode_main(g, pages, sinkwin, block_table, slot_ids, batch, hq, seq_lens,
                            sm_scale, num_workers, ws, stream);
}

hipError_t launch_int4_mfma_decode(const CacheGeom& g, const uint8_t* pages,
                                  const uint16_t* sinkwin, const int32_t* block_table,
                                  const int32_t* slot_ids, int batch, int hq, const uint16_t* q,
                                  const int32_t* seq_lens, const float* rot_k, float sm_scale,
                                  const Workspace& ws, hipStream_t stream) {
  if (batch == 0) return hipSuccess;
  const int G = hq / g.hkv;
  if (G != 1 && G != 2 && G != 4 && G != 8) return hipErrorInvalidValue;
  const int workers = G <= 4 ? int4_resident_workers<1>() : int4_resident_workers<8>();
  // Launch shape as for the INT2 pages (launch_decode).
  const int cus = current_device_cus();
  const bool small = (long long)batch * g.hkv * 2 < cus;
  const int window_first = small ? 1 : 0;
  const int wparts =
      small ? max(1, min(kWinSlots, (g.num_sink + g.window + kWinPartTokens - 1) / kWinPartTokens))
            : 1;
  const int hpw = small ? 1 : G;
  const hipError_t e = launch_prep_q_grid(dim3(g.hkv * (G / hpw), batch + 1), stream, g, q, rot_k,
                                          hq, seq_lens, workers, hpw, ws);
  if (e != hipSuccess) return e;
  const int worker_groups = (workers + kWaves - 1) / kWaves;
  const dim3 grid(worker_groups + batch * g.hkv * wparts);
  if (G <= 4)
    hipLaunchKernelGGL(int4_decode_mfma_kernel<1>, grid, dim3(64 * kWaves), 0, stream, g, pages,
                       sinkwin, block_table, slot_ids, hq, seq_lens, ws.plan(), sm_scale,
                       worker_groups, window_first, wparts, ws);
  else
    hipLaunchKernelGGL(int4_decode_mfma_kernel<8>, grid, dim3(64 * kWaves), 0, stream, g, pages,
                       sinkwin, block_table, slot_ids, hq, seq_lens, ws.plan(), sm_scale,
                       worker_groups, window_first, wparts, ws);
  return hipGetLastError();
}

}  // namespace oscar
