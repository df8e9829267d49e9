// Split combine: merge the per-split softmax partials of each (sequence, query head) in a fixed
// ascending order, normalise, and rotate the output back with the transpose of the value
// rotation (o = o' . R_V^T, exact for orthogonal R_V; OSCAR paper, "Abstract": fixed rotations
// keep attention aligned with what it consumes).
//
// One workgroup serves the G query heads of a KV head; every thread issues all of its global
// loads (its R_V row and its channel of every split) before the first use.
#include "oscar_internal.h"

namespace oscar {
namespace {

constexpr float kLn2 = 0.69314718055994531f;
constexpr int kRStride = kHeadDim + 4;  // floats per LDS row of R_V (16-byte aligned, skewed banks)

// grid (Hkv, batch), block 128 * G: thread (j, c) = (query head of the group, channel).
__global__ __launch_bounds__(1024) void combine_kernel(int hq, int hkv, Workspace ws,
                                                      const float* __restrict__ rot_v,
                                                      float* __restrict__ out,
                                                      float* __restrict__ lse) {
  const int h = blockIdx.x, b = blockIdx.y;
  const int G = hq / hkv;
  const int j = threadIdx.x >> 7, c = threadIdx.x & 127;
  const int ns = ws.nslots;
  const int jq = h * G + j;
  extern __shared__ float s_w[];        // [2][G][ns]: merge weights 2^(m - M) (0 for empty), l
  __shared__ __attribute__((aligned(16))) float s_o[8][kHeadDim];
  __shared__ float s_red[8][4];         // per head: max, then l, of each of its two waves
  __shared__ float4 s_r[kHeadDim][kRStride / 4];  // R_V[h], rows padded: conflict-free reads

  // Issue the loads first: R_V[h] (coalesced, into LDS) and this thread's channel of the slots.
  // Loads are issued 8 at a time before their LDS stores, so staging costs one memory latency
  // for G >= 4 (4096 quads over 512 or 1024 threads) and 2 or 4 for G = 2, 1.
  if (rot_v != nullptr) {
    const float4* R = reinterpret_cast<const float4*>(rot_v + (size_t)h * kHeadDim * kHeadDim);
    constexpr int kQuads = kHeadDim * kHeadDim / 4, kChunk = 8;
    for (int e0 = threadIdx.x; e0 < kQuads; e0 += kChunk * blockDim.x) {
      float4 rr[kChunk];
#pragma unroll
      for (int k = 0; k < kChunk; ++k) {
        const int e = e0 + k * blockDim.x;
        rr[k] = e < kQuads ? R[e] : make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
      for (int k = 0; k < kChunk; ++k) {
        const int e = e0 + k * blockDim.x;
        if (e < kQuads) s_r[e / (kHeadDim / 4)][e % (kHeadDim / 4)] = rr[k];
      }
    }
  }
  // INT2 partials in slots [0, nvalid), the BF16 sink/window partials in the last kWinSlots
  // slots.  All loads are issued before nvalid is known (slots past it hold stale but readable
  // values that never enter the sums), so the kernel pays one memory latency, not two.
  const int nv_raw = ws.nvalid()[b * hkv + h];
  const int ms = ws.max_splits();
  const float* o = ws.o(b, hq, jq, 0) + c;
  constexpr int kBatch = 16;
  float ov[kBatch];
#pragma unroll
  for (int e = 0; e < kBatch; ++e) ov[e] = e < ms ? o[(size_t)e * kHeadDim] : 0.f;
  float ow[kWinSlots];
#pragma unroll
  for (int k = 0; k < kWinSlots; ++k) ow[k] = o[(size_t)(ms + k) * kHeadDim];
  for (int e = c; e < ns; e += 128) {  // raw (m, l) of every slot of head j
    const float2 ml = *ws.ml(b, hq, jq, e);
    s_w[j * ns + e] = ml.x;
    s_w[G * ns + j * ns + e] = ml.y;
  }
  __syncthreads();
  const int nv = min(max(nv_raw, 0), ms);
  // Merge weights, computed by the head's 128 threads (entry e by thread e % 128): the INT2
  // slots 0 .. nv-1 and the window slots; M and l reduced in a fixed order.
  float* wm = s_w + j * ns;
  const float* wl = s_w + G * ns + j * ns;
  float mloc = -INFINITY;
  for (int e = c; e < ns; e += 128)
    if ((e < nv || e >= ms) && wl[e] > 0.f) mloc = fmaxf(mloc, wm[e]);
  for (int o2 = 32; o2 >= 1; o2 >>= 1) mloc = fmaxf(mloc, __shfl_xor(mloc, o2));
  if ((c & 63) == 0) s_red[j][c >> 6] = mloc;
  __syncthreads();
  const float M = fmaxf(s_red[j][0], s_red[j][1]);
  float lloc = 0.f;
  for (int e = c; e < ns; e += 128) {
    const bool use = (e < nv || e >= ms) && wl[e] > 0.f;
    const float w = use ? __builtin_amdgcn_exp2f(wm[e] - M) : 0.f;
    wm[e] = w;
    if (use) lloc = fmaf(w, wl[e], lloc);  // an unused slot's stale l may be NaN
  }
  for (int o2 = 32; o2 >= 1; o2 >>= 1) lloc += __shfl_xor(lloc, o2);
  if ((c & 63) == 0) s_red[j][2 + (c >> 6)] = lloc;
  __syncthreads();
  const float l = s_red[j][2] + s_red[j][3];
  const float inv = l > 0.f ? 1.0f / l : 0.f;
  if (c == 0 && lse != nullptr) lse[(size_t)b * hq + jq] = l > 0.f ? M * kLn2 + logf(l) : -INFINITY;
  // o'[j][c] = sum_e w_e o'_e[c] / l over the INT2 slots in order, then the window slots in
  // order; an empty entry (w = 0) is skipped, so its partial output is never read into the
  // sum.  Slots past the first 16 are loaded 16 at a time.
  const float* wj = wm;
  float acc = 0.f;
#pragma unroll
  for (int e = 0; e < kBatch; ++e) {
    if (e < nv && wj[e] > 0.f) acc = fmaf(wj[e], ov[e], acc);
  }
  for (int e0 = kBatch; e0 < nv; e0 += kBatch) {
    float ob[kBatch];
#pragma unroll
    for (int e = 0; e < kBatch; ++e) ob[e] = e0 + e < nv ? o[(size_t)(e0 + e) * kHeadDim] : 0.f;
#pragma unroll
    for (int e = 0; e < kBatch; ++e) {
      const float w = e0 + e < nv ? wj[e0 + e] : 0.f;
      if (w > 0.f) acc = fmaf(w, ob[e], acc);
    }
  }
#pragma unroll
  for (int k = 0; k < kWinSlots; ++k)
    if (wj[ms + k] > 0.f) acc = fmaf(wj[ms + k], ow[k], acc);
  s_o[j][c] = acc * inv;
  __syncthreads();
  float* orow = out + ((size_t)b * hq + jq) * kHeadDim;
  if (rot_v == nullptr) {
    orow[c] = s_o[j][c];
    return;
  }
  // out[j][c] = sum_k o'[j][k] * R_V[h][c][k]
  float acc2 = 0.f;
#pragma unroll 8
  for (int k4 = 0; k4 < kHeadDim / 4; ++k4) {
    const float4 r = s_r[c][k4];
    const float4 ov = *reinterpret_cast<const float4*>(&s_o[j][4 * k4]);
    acc2 = fmaf(ov.x, r.x, acc2);
    acc2 = fmaf(ov.y, r.y, acc2);
    acc2 = fmaf(ov.z, r.z, acc2);
    acc2 = fmaf(ov.w, r.w, acc2);
  }
  orow[c] = acc2;
}

// Small-grid form: grid (Hq, batch), block 512, one workgroup per query head, for launches
// where one workgroup per KV head would leave most of the chip idle and each head has many
// splits.  Thread t = (slot lane sg = t / 32 of 16, channel quad c4 = t % 32): slot lane sg
// sums slots sg, sg + 16, ... in ascending order with 16-byte loads; its first eight slots and
// the BF16 slot are loaded with everything else at the start (slots past the pair's count are
// read but never used), the rest eight at a time.  The 16 lanes' partial sums are added in lane
// order.  For R_V^T, thread t computes half (kh = t % 2) of output channel t / 2 (only threads
// < 256) from its R_V row, loaded first.
constexpr int kHeadThreads = 512, kSlotLanes = kHeadThreads / 32;
static_assert(kWinSlots <= kSlotLanes, "one slot lane per window slot");

__global__ __launch_bounds__(kHeadThreads) void combine_head_kernel(int hq, int hkv, Workspace ws,
                                                                  const float* __restrict__ rot_v,
                                                                  float* __restrict__ out,
                                                                  float* __restrict__ lse) {
  const int jq = blockIdx.x, b = blockIdx.y, h = jq / (hq / hkv);
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int ns = ws.nslots;
  extern __shared__ float s_w[];  // [2][ns]: m of each slot (then its merge weight), l
  __shared__ float4 s_part[kSlotLanes][32];
  __shared__ float4 s_win[kWinSlots][32];  // the window slots' outputs
  __shared__ float s_o[kHeadDim];
  __shared__ float s_red[2][kHeadThreads / 64];

  const int c_out = t >> 1, kh = t & 1;
  float4 r[16];
  if (rot_v != nullptr && t < 2 * kHeadDim) {
    const float4* R = reinterpret_cast<const float4*>(
        rot_v + ((size_t)h * kHeadDim + c_out) * kHeadDim + (kHeadDim / 2) * kh);
#pragma unroll
    for (int k = 0; k < 16; ++k) r[k] = R[k];
  }
  const int nv_raw = ws.nvalid()[b * hkv + h];
  const int sg = t >> 5, c4 = t & 31;
  const float4* ob = reinterpret_cast<const float4*>(ws.o(b, hq, jq, 0)) + c4;
  constexpr int kStride = kHeadDim / 4;  // float4 per slot
  constexpr int kFlight = 8;
  const int ms = ws.max_splits();
  float4 pre[kFlight];
#pragma unroll
  for (int k = 0; k < kFlight; ++k) {
    const int e = sg + k * kSlotLanes;
    pre[k] = e < ms ? ob[(size_t)e * kStride] : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  // window slot sg (< kWinSlots) of this thread's channel quad, added after the INT2 sums
  const float4 owin = sg < kWinSlots ? ob[(size_t)(ms + sg) * kStride] : make_float4(0.f, 0.f, 0.f, 0.f);
  for (int e = t; e < ns; e += kHeadThreads) {
    const float2 ml = *ws.ml(b, hq, jq, e);
    s_w[e] = ml.x;
    s_w[ns + e] = ml.y;
  }
  __syncthreads();
  const int nv = min(max(nv_raw, 0), ms);
  float* wm = s_w;
  const float* wl = s_w + ns;
  float mloc = -INFINITY;
  for (int e = t; e < ns; e += kHeadThreads)
    if ((e < nv || e >= ms) && wl[e] > 0.f) mloc = fmaxf(mloc, wm[e]);
  for (int o2 = 32; o2 >= 1; o2 >>= 1) mloc = fmaxf(mloc, __shfl_xor(mloc, o2));
  if (lane == 0) s_red[0][wv] = mloc;
  __syncthreads();
  float M = s_red[0][0];
#pragma unroll
  for (int k = 1; k < kHeadThreads / 64; ++k) M = fmaxf(M, s_red[0][k]);
  float lloc = 0.f;
  for (int e = t; e < ns; e += kHeadThreads) {
    const bool use = (e < nv || e >= ms) && wl[e] > 0.f;
    const float w = use ? __builtin_amdgcn_exp2f(wm[e] - M) : 0.f;
    wm[e] = w;
    if (use) lloc = fmaf(w, wl[e], lloc);  // an unused slot's stale l may be NaN
  }
  for (int o2 = 32; o2 >= 1; o2 >>= 1) lloc += __shfl_xor(lloc, o2);
  if (lane == 0) s_red[1][wv] = lloc;
  __syncthreads();
  float l = 0.f;
#pragma unroll
  for (int k = 0; k < kHeadThreads / 64; ++k) l += s_red[1][k];
  const float inv = l > 0.f ? 1.0f / l : 0.f;
  if (t == 0 && lse != nullptr) lse[(size_t)b * hq + jq] = l > 0.f ? M * kLn2 + logf(l) : -INFINITY;

  // o' partial sums: slot lane sg over slots sg, sg + 16, ... (< nv), skipping empty slots.
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  auto add = [&](float w, const float4& x) {
    if (w > 0.f) {
      acc.x = fmaf(w, x.x, acc.x);
      acc.y = fmaf(w, x.y, acc.y);
      acc.z = fmaf(w, x.z, acc.z);
      acc.w = fmaf(w, x.w, acc.w);
    }
  };
#pragma unroll
  for (int k = 0; k < kFlight; ++k) {
    const int e = sg + k * kSlotLanes;
    if (e < nv) add(wm[e], pre[k]);
  }
  int e = sg + kFlight * kSlotLanes;
  for (; e + (kFlight - 1) * kSlotLanes < nv; e += kFlight * kSlotLanes) {
    float4 x[kFlight];
#pragma unroll
    for (int k = 0; k < kFlight; ++k) x[k] = ob[(size_t)(e + k * kSlotLanes) * kStride];
#pragma unroll
    for (int k = 0; k < kFlight; ++k) add(wm[e + k * kSlotLanes], x[k]);
  }
  for (; e < nv; e += kSlotLanes) add(wm[e], ob[(size_t)e * kStride]);
  s_part[sg][c4] = acc;
  if (sg < kWinSlots) s_win[sg][c4] = owin;
  __syncthreads();
  if (t < 32) {
    float4 sum = s_part[0][t];
#pragma unroll
    for (int k = 1; k < kSlotLanes; ++k) {
      const float4 v = s_part[k][t];
      sum.x += v.x;
      sum.y += v.y;
      sum.z += v.z;
      sum.w += v.w;
    }
#pragma unroll
    for (int k = 0; k < kWinSlots; ++k) {
      const float ww = wm[ms + k];
      if (ww > 0.f) {
        const float4 x = s_win[k][t];
        sum.x = fmaf(ww, x.x, sum.x);
        sum.y = fmaf(ww, x.y, sum.y);
        sum.z = fmaf(ww, x.z, sum.z);
        sum.w = fmaf(ww, x.w, sum.w);
      }
    }
    s_o[4 * t + 0] = sum.x * inv;
    s_o[4 * t + 1] = sum.y * inv;
    s_o[4 * t + 2] = sum.z * inv;
    s_o[4 * t + 3] = sum.w * inv;
  }
  __syncthreads();
  float* orow = out + ((size_t)b * hq + jq) * kHeadDim;
  if (rot_v == nullptr) {
    if (t < kHeadDim) orow[t] = s_o[t];
    return;
  }
  if (t >= 2 * kHeadDim) return;
  // out[c] = sum_k o'[k] * R_V[h][c][k]: the two halves of k, then their sum (low half first)
  float part = 0.f;
#pragma unroll
  for (int k4 = 0; k4 < 16; ++k4) {
    const int k = (kHeadDim / 2) * kh + 4 * k4;
    part = fmaf(s_o[k + 0], r[k4].x, part);
    part = fmaf(s_o[k + 1], r[k4].y, part);
    part = fmaf(s_o[k + 2], r[k4].z, part);
    part = fmaf(s_o[k + 3], r[k4].w, part);
  }
  const float other = __shfl_xor(part, 1);
  if (kh == 0) orow[c_out] = part + other;
}

}  // namespace

hipError_t launch_combine(int batch, int hq, int hkv, const Workspace& ws, const float* rot_v,
                          float* out, float* lse, hipStream_t stream) {
  if (batch == 0) return hipSuccess;
  // One workgroup per query head when one per KV head would cover less than half of the
  // compute units and the heads have many splits to merge.
  const int cus = current_device_cus();
  if (cus <= 0) return hipErrorInvalidValue;
  if ((long long)batch * hkv * 2 < cus && ws.max_splits() > 32) {
    const size_t lds1 = (size_t)2 * ws.nslots * sizeof(float);
    hipLaunchKernelGGL(combine_head_kernel, dim3(hq, batch), dim3(kHeadThreads), lds1, stream, hq,
                       hkv, ws, rot_v, out, lse);
    return hipGetLastError();
  }
  const size_t lds = (size_t)2 * (hq / hkv) * ws.nslots * sizeof(float);
  if (lds > 48 * 1024) return hipErrorInvalidValue;
  hipLaunchKernelGGL(combine_kernel, dim3(hkv, batch), dim3(128 * (hq / hkv)), lds, stream, hq, hkv,
                     ws, rot_v, out, lse);
  return hipGetLastError();
}

}  // namespace oscar
