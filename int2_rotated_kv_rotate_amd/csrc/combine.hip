// Split combine: merge the per-split softmax partials of each (sequence, query head) in a fixed
// ascending order, normalise, and rotate the output back with the transpose of the value
// rotation (o = o' . R_V^T, exact for orthogonal R_V; OSCAR paper, "Abstract": fixed rotations
// keep attention aligned with what it consumes).
//
// Both forms issue their first loads together (R_V rows into registers, the first partial
// outputs, the (m, l) pairs), so a workgroup pays about one memory latency for most pairs, and
// need one workgroup barrier before the R_V^T product (the per-query-head form two more).
// R_V^T: thread (row c, part p) of 8 threads per row holds R_V[h][c][k] for the p-th slice of
// 16 k in registers, sums o'[k] R_V[h][c][k] over its slice in ascending k, and the 8 slices
// are added by a butterfly over the 8 adjacent lanes (a fixed order).  Lane reductions use DPP
// row operations and lane reads, not LDS permutes.
#include "oscar_internal.h"

namespace oscar {
namespace {

constexpr float kLn2 = 0.69314718055994531f;

// DPP lane moves within rows of 16 lanes: quad_perm xor 1 and xor 2, row rotation by 8 (= xor
// 8), and xor 4 from a left and a right row shift on alternate banks of 4 lanes.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                               0xF, 0xF, false));
}
constexpr int kXor1 = 0xB1, kXor2 = 0x4E, kRor8 = 0x128;
__device__ __forceinline__ float xor4(float v) {
  const int x = __builtin_bit_cast(int, v);
  int t = __builtin_amdgcn_update_dpp(x, x, 0x104, 0xF, 0x5, false);  // row_shl:4, banks 0, 2
  t = __builtin_amdgcn_update_dpp(t, x, 0x114, 0xF, 0xA, false);      // row_shr:4, banks 1, 3
  return __builtin_bit_cast(float, t);
}
// Sum / max over the 16 lanes of each row: every lane of a row gets the same value.
__device__ __forceinline__ float row_sum(float v) {
  v += dpp<kXor1>(v);
  v += dpp<kXor2>(v);
  v += xor4(v);
  return v + dpp<kRor8>(v);
}
__device__ __forceinline__ float row_max(float v) {
  v = fmaxf(v, dpp<kXor1>(v));
  v = fmaxf(v, dpp<kXor2>(v));
  v = fmaxf(v, xor4(v));
  return fmaxf(v, dpp<kRor8>(v));
}
__device__ __forceinline__ float lane_value(float v, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}
__device__ __forceinline__ float wave_sum(float v) {
  v = row_sum(v);
  return (lane_value(v, 0) + lane_value(v, 16)) + (lane_value(v, 32) + lane_value(v, 48));
}
__device__ __forceinline__ float wave_max(float v) {
  v = row_max(v);
  return fmaxf(fmaxf(lane_value(v, 0), lane_value(v, 16)),
               fmaxf(lane_value(v, 32), lane_value(v, 48)));
}

// A slot enters the merge if it is one of the pair's INT2 slots (e < nv) or a window slot
// (e >= ms) and holds positions (l > 0); the outputs of other slots are never read into a sum
// (their stale values may be NaN).
__device__ __forceinline__ bool slot_used(int e, int nv, int ms, float l) {
  return (e < nv || e >= ms) && l > 0.f;
}

// R_V^T: 8 threads per output row.
constexpr int kRotParts = 8, kRotQuads = kHeadDim / 4 / kRotParts;

// R_V[h] row c, slice part: kRotQuads float4, loaded first and used last.
__device__ __forceinline__ void load_rot(const float* rot_v, int h, int c, int part,
                                         float4 (&r)[kRotQuads]) {
  const float4* R =
      reinterpret_cast<const float4*>(rot_v + ((size_t)h * kHeadDim + c) * kHeadDim) +
      part * kRotQuads;
#pragma unroll
  for (int i = 0; i < kRotQuads; ++i) r[i] = R[i];
}

// o'[k] R_V[c][k] over the thread's slice (k ascending) for the o' row so, then the 8 slices of
// the row added by a butterfly over the 8 adjacent lanes: every lane of the 8 gets the sum.
__device__ __forceinline__ float rot_slice(const float* so, const float4 (&r)[kRotQuads], int part) {
  const float4* s4 = reinterpret_cast<const float4*>(so) + part * kRotQuads;
  float acc = 0.f;
#pragma unroll
  for (int i = 0; i < kRotQuads; ++i) {
    const float4 x = s4[i];
    acc = fmaf(x.x, r[i].x, acc);
    acc = fmaf(x.y, r[i].y, acc);
    acc = fmaf(x.z, r[i].z, acc);
    acc = fmaf(x.w, r[i].w, acc);
  }
  acc += dpp<kXor1>(acc);
  acc += dpp<kXor2>(acc);
  return acc + xor4(acc);
}

// Query-head rows per workgroup of the per-KV-head form: 8 / G sequences x G heads, so R_V[h]
// is read once for 8 rows whatever G is.
constexpr int kRows = 8, kRowThreads = kRows * kHeadDim;

// grid (Hkv, ceil(batch / (8 / G))), block 1024.
// Merge role: thread (row j, channel c), row j = (sequence b0 + j / G, head j % G of the
// group); each of a row's two wavefronts computes the row's merge weights itself (max and sum
// in a fixed order, every lane holding the weights of slots lane, lane + 64) and reads a
// slot's weight with a lane read, so the merge needs no barrier and no LDS.
// R_V^T role: every thread, (output row u / 8, slice u % 8), for the 8 o' rows.
__global__ __launch_bounds__(kRowThreads) void combine_kernel(int batch, int hq, int hkv,
                                                            Workspace ws,
                                                            const float* __restrict__ rot_v,
                                                            float* __restrict__ out,
                                                            float* __restrict__ lse) {
  const int h = blockIdx.x;
  const int G = hq / hkv, nb = kRows / G;
  const int u = threadIdx.x, lane = u & 63;
  const int j = u >> 7, c = u & 127;
  const int b = blockIdx.y * nb + j / G, jq = h * G + j % G;
  const bool live = b < batch;  // uniform per wavefront
  const int ns = ws.nslots, ms = ws.max_splits();
  __shared__ __attribute__((aligned(16))) float s_o[kRows][kHeadDim];

  float4 r[kRotQuads];
  if (rot_v != nullptr) load_rot(rot_v, h, u / kRotParts, u % kRotParts, r);
  // The first kFirst INT2 slots and window slot 0 are loaded with everything else; later INT2
  // slots (past kFirst, up to nv) kBatch at a time, and window slots 1.. only where used.
  constexpr int kFirst = 12, kBatch = 8;
  constexpr int kMl = 2;  // (m, l) of slots lane and lane + 64, loaded up front
  if (live) {
    const int nv = min(max(ws.nvalid()[b * hkv + h], 0), ms);
    const float* o = ws.o(b, hq, jq, 0) + c;
    float ov[kFirst];
#pragma unroll
    for (int e = 0; e < kFirst; ++e) ov[e] = e < ms ? o[(size_t)e * kHeadDim] : 0.f;
    const float ow0 = o[(size_t)ms * kHeadDim];
    float2 mlr[kMl];
#pragma unroll
    for (int i = 0; i < kMl; ++i) {
      const int e = lane + 64 * i;
      mlr[i] = e < ns ? *ws.ml(b, hq, jq, e) : make_float2(-INFINITY, 0.f);
    }
    // M over the used slots, then w_e = 2^(m_e - M) and l = sum_e w_e l_e (lane sums in slot
    // order, then the fixed reduction)
    float mloc = -INFINITY;
#pragma unroll
    for (int i = 0; i < kMl; ++i) {
      const int e = lane + 64 * i;
      if (e < ns && slot_used(e, nv, ms, mlr[i].y)) mloc = fmaxf(mloc, mlr[i].x);
    }
    for (int e = lane + 64 * kMl; e < ns; e += 64) {
      const float2 ml = *ws.ml(b, hq, jq, e);
      if (slot_used(e, nv, ms, ml.y)) mloc = fmaxf(mloc, ml.x);
    }
    const float M = wave_max(mloc);
    float wl[kMl];  // weights of slots lane, lane + 64
    float lloc = 0.f;
#pragma unroll
    for (int i = 0; i < kMl; ++i) {
      const int e = lane + 64 * i;
      const bool use = e < ns && slot_used(e, nv, ms, mlr[i].y);
      wl[i] = use ? __builtin_amdgcn_exp2f(mlr[i].x - M) : 0.f;
      if (use) lloc = fmaf(wl[i], mlr[i].y, lloc);
    }
    for (int e = lane + 64 * kMl; e < ns; e += 64) {
      const float2 ml = *ws.ml(b, hq, jq, e);
      if (slot_used(e, nv, ms, ml.y)) lloc = fmaf(__builtin_amdgcn_exp2f(ml.x - M), ml.y, lloc);
    }
    const float l = wave_sum(lloc);
    const float inv = l > 0.f ? 1.0f / l : 0.f;
    if (c == 0 && lse != nullptr) lse[(size_t)b * hq + jq] = l > 0.f ? M * kLn2 + logf(l) : -INFINITY;
    // weight of slot e (uniform): from the lane that holds it, else from its (m, l)
    auto weight = [&](int e) {
      if (e < 64 * kMl) return lane_value(e < 64 ? wl[0] : wl[1], e & 63);
      const float2 ml = *ws.ml(b, hq, jq, e);
      return slot_used(e, nv, ms, ml.y) ? __builtin_amdgcn_exp2f(ml.x - M) : 0.f;
    };
    // used window slots past the first: their loads go out before the INT2 sums
    float owk[kWinSlots - 1];
#pragma unroll
    for (int k = 1; k < kWinSlots; ++k)
      owk[k - 1] = weight(ms + k) > 0.f ? o[(size_t)(ms + k) * kHeadDim] : 0.f;
    // o'[j][c] = sum_e w_e o'_e[c] / l: INT2 slots in order, then the window slots in order
    float acc = 0.f;
#pragma unroll
    for (int e = 0; e < kFirst; ++e) {
      if (e < nv) {
        const float w = weight(e);
        if (w > 0.f) acc = fmaf(w, ov[e], acc);
      }
    }
    for (int e0 = kFirst; e0 < nv; e0 += kBatch) {
      float ob[kBatch];
#pragma unroll
      for (int e = 0; e < kBatch; ++e) ob[e] = e0 + e < nv ? o[(size_t)(e0 + e) * kHeadDim] : 0.f;
#pragma unroll
      for (int e = 0; e < kBatch; ++e) {
        if (e0 + e < nv) {
          const float w = weight(e0 + e);
          if (w > 0.f) acc = fmaf(w, ob[e], acc);
        }
      }
    }
    {
      const float w = weight(ms);
      if (w > 0.f) acc = fmaf(w, ow0, acc);
    }
#pragma unroll
    for (int k = 1; k < kWinSlots; ++k) {
      const float w = weight(ms + k);
      if (w > 0.f) acc = fmaf(w, owk[k - 1], acc);
    }
    s_o[j][c] = acc * inv;
  }
  __syncthreads();
  if (rot_v == nullptr) {
    if (live) out[((size_t)b * hq + jq) * kHeadDim + c] = s_o[j][c];
    return;
  }
  // out[row jr][c'] = sum_k o'[jr][k] R_V[h][c'][k]; lane slice p writes row p
  const int crow = u / kRotParts, part = u % kRotParts;
  const int b0 = blockIdx.y * nb;
#pragma unroll
  for (int jr = 0; jr < kRows; ++jr) {
    const int br = b0 + jr / G;
    if (br < batch) {  // uniform
      const float v = rot_slice(s_o[jr], r, part);
      if (part == jr) out[((size_t)br * hq + h * G + jr % G) * kHeadDim + crow] = v;
    }
  }
}

// Per-query-head form: grid (Hq, batch), block 1024, for launches where one workgroup per KV
// head would leave most of the chip idle and each head has many splits.
//   (m, l) role: thread u takes slots u, u + 1024, ... with a running (max, sum); the
//     wavefronts' pairs are merged through LDS (one barrier) in wavefront order.
//   slot lanes: thread (sg = u / 32 of 32, channel quad u % 32) sums slots sg, sg + 32, ... in
//     ascending order with 16-byte loads, the first eight loaded at the start, the rest eight
//     at a time; then (second barrier) thread ch < 128 adds the 32 lanes' sums in lane order,
//     then the window slots in order.
//   R_V^T: thread (row u / 8, slice u % 8), its 16 values of R_V[h][row] loaded at the start.
// The (m, l) merges of a wavefront run over its rows of 16 lanes, then its four rows in order.
constexpr int kHeadThreads = 1024, kSlotLanes = kHeadThreads / 32, kHeadWaves = kHeadThreads / 64;
static_assert(kWinSlots <= kSlotLanes, "one slot lane per window slot");

__global__ __launch_bounds__(kHeadThreads) void combine_head_kernel(int hq, int hkv, Workspace ws,
                                                                  const float* __restrict__ rot_v,
                                                                  float* __restrict__ out,
                                                                  float* __restrict__ lse) {
  const int jq = blockIdx.x, b = blockIdx.y, h = jq / (hq / hkv);
  const int u = threadIdx.x, lane = u & 63, wv = u >> 6;
  const int ns = ws.nslots, ms = ws.max_splits();
  extern __shared__ float s_m[];  // [ns]: m of each used slot, -inf for the others
  __shared__ __attribute__((aligned(16))) float s_part[kSlotLanes][kHeadDim];
  __shared__ __attribute__((aligned(16))) float s_win[kWinSlots][kHeadDim];
  __shared__ __attribute__((aligned(16))) float s_o[kHeadDim];
  __shared__ float2 s_red[kHeadWaves];

  float4 r[kRotQuads];
  if (rot_v != nullptr) load_rot(rot_v, h, u / kRotParts, u % kRotParts, r);
  const int nv = min(max(ws.nvalid()[b * hkv + h], 0), ms);
  const int sg = u >> 5, c4 = u & 31;
  const float4* ob = reinterpret_cast<const float4*>(ws.o(b, hq, jq, 0)) + c4;
  constexpr int kStride = kHeadDim / 4;  // float4 per slot
  constexpr int kFlight = 8;
  float4 pre[kFlight];
#pragma unroll
  for (int k = 0; k < kFlight; ++k) {
    const int e = sg + k * kSlotLanes;
    pre[k] = e < ms ? ob[(size_t)e * kStride] : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  // window slot sg (< kWinSlots) of this thread's channel quad
  const float4 owin = sg < kWinSlots ? ob[(size_t)(ms + sg) * kStride] : make_float4(0.f, 0.f, 0.f, 0.f);
  const float2 ml0 = u < ns ? *ws.ml(b, hq, jq, u) : make_float2(-INFINITY, 0.f);

  // running (max, sum of 2^(m - max) l) over this thread's slots, then the wavefront's
  float mt = -INFINITY, lt = 0.f;
  auto take = [&](int e, float2 ml) {
    const bool use = slot_used(e, nv, ms, ml.y);
    s_m[e] = use ? ml.x : -INFINITY;
    if (use) {
      if (ml.x > mt) {
        lt = lt * __builtin_amdgcn_exp2f(mt - ml.x) + ml.y;
        mt = ml.x;
      } else {
        lt = fmaf(__builtin_amdgcn_exp2f(ml.x - mt), ml.y, lt);
      }
    }
  };
  if (u < ns) take(u, ml0);
  for (int e = u + kHeadThreads; e < ns; e += kHeadThreads) take(e, *ws.ml(b, hq, jq, e));
  // (max, sum) pairs merged over each row of 16 lanes, then the four rows in order
  auto merge_pair = [&](float m2, float l2) {
    const float mm = fmaxf(mt, m2);
    float ln = 0.f;
    if (mt > -INFINITY) ln = lt * __builtin_amdgcn_exp2f(mt - mm);
    if (m2 > -INFINITY) ln = fmaf(l2, __builtin_amdgcn_exp2f(m2 - mm), ln);
    mt = mm;
    lt = ln;
  };
  merge_pair(dpp<kXor1>(mt), dpp<kXor1>(lt));
  merge_pair(dpp<kXor2>(mt), dpp<kXor2>(lt));
  merge_pair(xor4(mt), xor4(lt));
  merge_pair(dpp<kRor8>(mt), dpp<kRor8>(lt));
  {
    const float m0 = lane_value(mt, 0), l0 = lane_value(lt, 0);
    const float m1 = lane_value(mt, 16), l1 = lane_value(lt, 16);
    const float m2 = lane_value(mt, 32), l2 = lane_value(lt, 32);
    const float m3 = lane_value(mt, 48), l3 = lane_value(lt, 48);
    mt = m0;
    lt = l0;
    merge_pair(m1, l1);
    merge_pair(m2, l2);
    merge_pair(m3, l3);
  }
  if (lane == 0) s_red[wv] = make_float2(mt, lt);
  // slot lanes' channel quads and the window slots' outputs go to LDS after the barrier
  __syncthreads();
  float M = -INFINITY;
#pragma unroll
  for (int k = 0; k < kHeadWaves; ++k) M = fmaxf(M, s_red[k].x);
  float l = 0.f;
#pragma unroll
  for (int k = 0; k < kHeadWaves; ++k) {
    const float2 p = s_red[k];
    if (p.x > -INFINITY) l = fmaf(p.y, __builtin_amdgcn_exp2f(p.x - M), l);
  }
  const float inv = l > 0.f ? 1.0f / l : 0.f;
  if (u == 0 && lse != nullptr) lse[(size_t)b * hq + jq] = l > 0.f ? M * kLn2 + logf(l) : -INFINITY;

  // o' partial sums: slot lane sg over slots sg, sg + 32, ... (< nv), skipping unused slots
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  auto add = [&](int e, const float4& x) {
    const float me = s_m[e];
    if (me > -INFINITY) {
      const float w = __builtin_amdgcn_exp2f(me - M);
      acc.x = fmaf(w, x.x, acc.x);
      acc.y = fmaf(w, x.y, acc.y);
      acc.z = fmaf(w, x.z, acc.z);
      acc.w = fmaf(w, x.w, acc.w);
    }
  };
#pragma unroll
  for (int k = 0; k < kFlight; ++k) {
    const int e = sg + k * kSlotLanes;
    if (e < nv) add(e, pre[k]);
  }
  int e = sg + kFlight * kSlotLanes;
  for (; e + (kFlight - 1) * kSlotLanes < nv; e += kFlight * kSlotLanes) {
    float4 x[kFlight];
#pragma unroll
    for (int k = 0; k < kFlight; ++k) x[k] = ob[(size_t)(e + k * kSlotLanes) * kStride];
#pragma unroll
    for (int k = 0; k < kFlight; ++k) add(e + k * kSlotLanes, x[k]);
  }
  for (; e < nv; e += kSlotLanes) add(e, ob[(size_t)e * kStride]);
  reinterpret_cast<float4*>(s_part[sg])[c4] = acc;
  if (sg < kWinSlots) reinterpret_cast<float4*>(s_win[sg])[c4] = owin;
  __syncthreads();
  if (u < kHeadDim) {
    float sum = s_part[0][u];
#pragma unroll
    for (int k = 1; k < kSlotLanes; ++k) sum += s_part[k][u];
#pragma unroll
    for (int k = 0; k < kWinSlots; ++k) {
      const float me = s_m[ms + k];
      if (me > -INFINITY) sum = fmaf(__builtin_amdgcn_exp2f(me - M), s_win[k][u], sum);
    }
    s_o[u] = sum * inv;
  }
  __syncthreads();
  float* orow = out + ((size_t)b * hq + jq) * kHeadDim;
  if (rot_v == nullptr) {
    if (u < kHeadDim) orow[u] = s_o[u];
    return;
  }
  const float v = rot_slice(s_o, r, u % kRotParts);
  if (u % kRotParts == 0) orow[u / kRotParts] = v;
}

}  // namespace

hipError_t launch_combine(int batch, int hq, int hkv, const Workspace& ws, const float* rot_v,
                          float* out, float* lse, hipStream_t stream) {
  if (batch == 0) return hipSuccess;
  // One workgroup per query head when the (sequence, KV head) pairs would cover less than half
  // of the compute units and the heads have many splits to merge; else 8 query-head rows of
  // one KV head per workgroup.
  const int cus = current_device_cus();
  if (cus <= 0) return hipErrorInvalidValue;
  if ((long long)batch * hkv * 2 < cus && ws.max_splits() > 32) {
    const size_t lds1 = (size_t)ws.nslots * sizeof(float);
    hipLaunchKernelGGL(combine_head_kernel, dim3(hq, batch), dim3(kHeadThreads), lds1, stream, hq,
                       hkv, ws, rot_v, out, lse);
    return hipGetLastError();
  }
  const int nb = kRows / (hq / hkv);
  hipLaunchKernelGGL(combine_kernel, dim3(hkv, (batch + nb - 1) / nb), dim3(kRowThreads), 0, stream,
                     batch, hq, hkv, ws, rot_v, out, lse);
  return hipGetLastError();
}

}  // namespace oscar
