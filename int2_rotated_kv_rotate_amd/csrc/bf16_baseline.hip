// BF16 paged KV cache baseline: append (copy into pages) and split-K decode attention with the
// same work decomposition and partial format as the INT2 path, so both finish through the same
// combine kernel.  The method's memory, throughput and latency claims are all stated against a
// BF16 KV cache (write-up "OSCAR: Cut LLM Inference Costs 8x with 2-bit KV Cache Quantization",
// "Practical Summary"; OSCAR paper, "Abstract").
//
// Page (per physical page and KV head, 8192 bytes): K bf16 [16 tokens][128], then V transposed
// as bf16 [128 channels][16 tokens], so both MFMA operands load contiguous lane chunks.
#include "oscar_internal.h"

namespace oscar {
namespace {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef short v4s __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegBig = -1.0e30f;

// grid (total_new, Hkv), block 128 (thread = channel).
__global__ __launch_bounds__(128) void bf16_append_kernel(
    CacheGeom g, uint16_t* __restrict__ pages, const int32_t* __restrict__ block_table, int batch,
    const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
    const int32_t* __restrict__ new_offsets, const int32_t* __restrict__ start_pos) {
  const int n = blockIdx.x, h = blockIdx.y, c = threadIdx.x;
  const int b = row_to_seq(new_offsets, batch, n);
  const int pos = start_pos[b] + (n - new_offsets[b]);
  const int lp = pos / kPage;
  if (pos < 0 || lp >= g.max_pages) return;
  const int page = block_table[(size_t)b * g.max_pages + lp];
  if (page < 0 || page >= g.num_pages) return;
  uint16_t* pg = pages + ((size_t)page * g.hkv + h) * kBf16PageElems;
  const size_t src = ((size_t)n * g.hkv + h) * kHeadDim + c;
  const int r = pos % kPage;
  pg[r * kHeadDim + c] = k_new[src];
  pg[kPage * kHeadDim + c * kPage + r] = v_new[src];
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

// grid (max_splits, Hkv, batch), block 64.  Lane (kq = lane/16, c16 = lane%16).
// QK: S^T[t][j] = K[t][:] . q[j][:]; the K axis of MFMA kc, lane quarter kq, slot s is channel
// 32*kq + 4*kc + s (same on both operands).  PV: O[j][c] = P[j][t] V[t][c], tokens 4*kq + s.
__global__ __launch_bounds__(64) void bf16_decode_kernel(
    CacheGeom g, const uint16_t* __restrict__ pages, const int32_t* __restrict__ block_table,
    int hq, const uint16_t* __restrict__ q, const int32_t* __restrict__ seq_lens, float sm_scale,
    int split_pages, Workspace ws) {
  const int lane = threadIdx.x, kq = lane >> 4, c16 = lane & 15;
  const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int max_splits = ws.max_splits();
  const int G = hq / g.hkv;
  if (split == 0) {  // no sink/window split here: the pair's window slots are empty, and every
                     // split slot is written (each split writes its own, empty or not)
    static_assert(8 * kWinSlots <= 64, "one lane per window slot of the pair's heads");
    if (lane < G * kWinSlots)
      *ws.ml(b, hq, h * G + lane / kWinSlots, ws.win_slot() + lane % kWinSlots) =
          make_float2(kNegBig, 0.f);
    if (lane == 0) ws.nvalid()[b * g.hkv + h] = max_splits;
  }
  const int L = max(seq_lens[b], 0);
  const float sm_log2 = sm_scale * kLog2e;
  int pg0 = split * split_pages;
  int pg1 = (split == max_splits - 1) ? 0x7fffffff : pg0 + split_pages;
  pg1 = min(min(pg1, (L + kPage - 1) / kPage), g.max_pages);

  // q^T operand: column j = c16 (zero for j >= G), slots = channels 32*kq + 4*kc + s.
  v4s qb[8];
  {
    const bool jv = c16 < G;
    const uint16_t* qrow = q + ((size_t)b * hq + h * G + (jv ? c16 : 0)) * kHeadDim + 32 * kq;
    const uint4 a = reinterpret_cast<const uint4*>(qrow)[0];
    const uint4 bq = reinterpret_cast<const uint4*>(qrow)[1];
    const uint4 cq = reinterpret_cast<const uint4*>(qrow)[2];
    const uint4 dq = reinterpret_cast<const uint4*>(qrow)[3];
    const uint32_t w[16] = {a.x, a.y, a.z, a.w, bq.x, bq.y, bq.z, bq.w,
                            cq.x, cq.y, cq.z, cq.w, dq.x, dq.y, dq.z, dq.w};
#pragma unroll
    for (int kc = 0; kc < 8; ++kc) {
      const uint32_t lo = jv ? w[2 * kc] : 0u, hi = jv ? w[2 * kc + 1] : 0u;
      qb[kc] = (v4s){(short)(lo & 0xFFFF), (short)(lo >> 16), (short)(hi & 0xFFFF), (short)(hi >> 16)};
    }
  }

  v4f acc[8];
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) acc[nb] = (v4f){0.f, 0.f, 0.f, 0.f};
  float mrun = kNegBig, lsum = 0.f;
  const int32_t* bt = block_table + (size_t)b * g.max_pages;
  // Software pipeline: page pg is computed while page pg + 1's K and V are in flight and page
  // pg + 2's id is being fetched.  An id outside the pool skips its page.
  auto valid_id = [&](int id) { return id >= 0 && id < g.num_pages; };
  auto fetch = [&](int id, uint4 (&kk)[4], uint2 (&vv)[8]) {
    const uint16_t* base = pages + ((size_t)id * g.hkv + h) * kBf16PageElems;
    const uint4* krow = reinterpret_cast<const uint4*>(base + c16 * kHeadDim + 32 * kq);
#pragma unroll
    for (int k = 0; k < 4; ++k) kk[k] = krow[k];
    const uint16_t* vt = base + kPage * kHeadDim;
#pragma unroll
    for (int nb = 0; nb < 8; ++nb)
      vv[nb] = *reinterpret_cast<const uint2*>(vt + (16 * nb + c16) * kPage + 4 * kq);
  };
  uint4 kc[4] = {};
  uint2 vc[8] = {};
  int id_cur = pg0 < pg1 ? bt[pg0] : -1;
  int id_next = pg0 + 1 < pg1 ? bt[pg0 + 1] : -1;
  if (valid_id(id_cur)) fetch(id_cur, kc, vc);
  for (int pg = pg0; pg < pg1; ++pg) {
    uint4 kn[4] = {};
    uint2 vn[8] = {};
    if (pg + 1 < pg1 && valid_id(id_next)) fetch(id_next, kn, vn);
    const int id_after = pg + 2 < pg1 ? bt[pg + 2] : -1;
    if (valid_id(id_cur)) {
      const uint32_t kw[16] = {kc[0].x, kc[0].y, kc[0].z, kc[0].w, kc[1].x, kc[1].y, kc[1].z, kc[1].w,
                               kc[2].x, kc[2].y, kc[2].z, kc[2].w, kc[3].x, kc[3].y, kc[3].z, kc[3].w};
      v4f s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kc8 = 0; kc8 < 8; ++kc8) {
        const v4s ka = (v4s){(short)(kw[2 * kc8] & 0xFFFF), (short)(kw[2 * kc8] >> 16),
                             (short)(kw[2 * kc8 + 1] & 0xFFFF), (short)(kw[2 * kc8 + 1] >> 16)};
        s = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ka, qb[kc8], s, 0, 0, 0);
      }
      float lg[4];
      float tm = -INFINITY;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int pos = pg * kPage + 4 * kq + i;
        lg[i] = pos < L ? s[i] * sm_log2 : -INFINITY;
        tm = fmaxf(tm, lg[i]);
      }
      tm = fmaxf(tm, __shfl_xor(tm, 16));
      tm = fmaxf(tm, __shfl_xor(tm, 32));
      const float mnew = fmaxf(mrun, tm);
      if (__any(mnew > mrun)) {
        const float alpha = __builtin_amdgcn_exp2f(mrun - mnew);
        lsum *= alpha;
        // accumulator rows are query heads 4*kq + i: fetch their alphas from lanes 4*kq + i
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float ai = __shfl(alpha, 4 * kq + i);
#pragma unroll
          for (int nb = 0; nb < 8; ++nb) acc[nb][i] *= ai;
        }
        mrun = mnew;
      }
      float p[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[i] = lg[i] != -INFINITY ? __builtin_amdgcn_exp2f(lg[i] - mrun) : 0.f;
        lsum += p[i];
      }
      uint32_t h01, h23, l01, l23;
      split_bf16(p, h01, h23, l01, l23);
      const v4s ahi = (v4s){(short)(h01 & 0xFFFF), (short)(h01 >> 16), (short)(h23 & 0xFFFF), (short)(h23 >> 16)};
      const v4s alo = (v4s){(short)(l01 & 0xFFFF), (short)(l01 >> 16), (short)(l23 & 0xFFFF), (short)(l23 >> 16)};
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) {
        const uint2 vv = vc[nb];
        const v4s vb = (v4s){(short)(vv.x & 0xFFFF), (short)(vv.x >> 16), (short)(vv.y & 0xFFFF), (short)(vv.y >> 16)};
        acc[nb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ahi, vb, acc[nb], 0, 0, 0);
        acc[nb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(alo, vb, acc[nb], 0, 0, 0);
      }
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) kc[k] = kn[k];
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) vc[nb] = vn[nb];
    id_cur = pg + 1 < pg1 ? id_next : -1;
    id_next = id_after;
  }
  // l per query head j = c16 (sum over token quarters); rows of acc are heads 4*kq + i.
  const float lt = lsum + __shfl_xor(lsum, 16) + __shfl_xor(lsum, 32) + __shfl_xor(lsum, 48);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int j = 4 * kq + i;
    if (j < G) {
      float* o = ws.o(b, hq, h * G + j, split);
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) o[16 * nb + c16] = acc[nb][i];
    }
  }
  if (kq == 0 && c16 < G) *ws.ml(b, hq, h * G + c16, split) = make_float2(mrun, lt);
}

}  // namespace

hipError_t launch_bf16_append(const CacheGeom& g, uint16_t* pages, const int32_t* block_table,
                              int batch, int total_new, const uint16_t* k_new,
                              const uint16_t* v_new, const int32_t* new_offsets,
                              const int32_t* start_pos, hipStream_t stream) {
  if (batch == 0 || total_new == 0) return hipSuccess;
  hipLaunchKernelGGL(bf16_append_kernel, dim3(total_new, g.hkv), dim3(128), 0, stream, g, pages,
                     block_table, batch, k_new, v_new, new_offsets, start_pos);
  return hipGetLastError();
}

hipError_t launch_bf16_decode(const CacheGeom& g, const uint16_t* pages,
                              const int32_t* block_table, int batch, int hq, const uint16_t* q,
                              const int32_t* seq_lens, float sm_scale, int split_pages,
                              const Workspace& ws, hipStream_t stream) {
  if (batch == 0) return hipSuccess;
  hipLaunchKernelGGL(bf16_decode_kernel, dim3(ws.max_splits(), g.hkv, batch), dim3(64), 0, stream,
                     g, pages, block_table, hq, q, seq_lens, sm_scale, split_pages, ws);
  return hipGetLastError();
}

}  // namespace oscar
