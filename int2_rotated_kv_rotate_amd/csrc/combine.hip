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
  __shared__ float s_o[8][kHeadDim];
  __shared__ float s_red[8][4];         // per head: max, then l, of each of its two waves
  __shared__ float4 s_r[kHeadDim][kRStride / 4];  // R_V[h], rows padded: conflict-free reads

  // Issue the loads first: R_V[h] (coalesced, into LDS) and this thread's channel of the slots.
  // Loads are issued 4 at a time before their LDS stores (4096 quads = a multiple of
  // 4 * blockDim.x for every group size), so staging costs 1 to 8 memory latencies.
  if (rot_v != nullptr) {
    const float4* R = reinterpret_cast<const float4*>(rot_v + (size_t)h * kHeadDim * kHeadDim);
    constexpr int kQuads = kHeadDim * kHeadDim / 4, kChunk = 4;
    for (int e0 = threadIdx.x; e0 < kQuads; e0 += kChunk * blockDim.x) {
      float4 rr[kChunk];
#pragma unroll
      for (int k = 0; k < kChunk; ++k) rr[k] = R[e0 + k * blockDim.x];
#pragma unroll
      for (int k = 0; k < kChunk; ++k) {
        const int e = e0 + k * blockDim.x;
        s_r[e / (kHeadDim / 4)][e % (kHeadDim / 4)] = rr[k];
      }
    }
  }
  // INT2 partials in slots [0, nvalid), the BF16 sink/window partial in the last slot.  All
  // loads are issued before nvalid is known (slots past it hold stale but readable values that
  // never enter the sums), so the kernel pays one memory latency, not two.
  const int nv_raw = ws.nvalid()[b * hkv + h];
  const float* o = ws.o(b, hq, jq, 0) + c;
  constexpr int kBatch = 16;
  float ov[kBatch];
#pragma unroll
  for (int e = 0; e < kBatch; ++e) ov[e] = e < ns - 1 ? o[(size_t)e * kHeadDim] : 0.f;
  const float ow = o[(size_t)(ns - 1) * kHeadDim];
  for (int e = c; e < ns; e += 128) {  // raw (m, l) of every slot of head j
    const float2 ml = *ws.ml(b, hq, jq, e);
    s_w[j * ns + e] = ml.x;
    s_w[G * ns + j * ns + e] = ml.y;
  }
  __syncthreads();
  const int nv = min(max(nv_raw, 0), ns - 1);
  // Merge weights, computed by the head's 128 threads (entry e by thread e % 128): the INT2
  // slots 0 .. nv-1 and the window slot; M and l reduced in a fixed order.
  float* wm = s_w + j * ns;
  const float* wl = s_w + G * ns + j * ns;
  float mloc = -INFINITY;
  for (int e = c; e < ns; e += 128)
    if ((e < nv || e == ns - 1) && wl[e] > 0.f) mloc = fmaxf(mloc, wm[e]);
  for (int o2 = 32; o2 >= 1; o2 >>= 1) mloc = fmaxf(mloc, __shfl_xor(mloc, o2));
  if ((c & 63) == 0) s_red[j][c >> 6] = mloc;
  __syncthreads();
  const float M = fmaxf(s_red[j][0], s_red[j][1]);
  float lloc = 0.f;
  for (int e = c; e < ns; e += 128) {
    const bool use = (e < nv || e == ns - 1) && wl[e] > 0.f;
    const float w = use ? __builtin_amdgcn_exp2f(wm[e] - M) : 0.f;
    wm[e] = w;
    lloc = fmaf(w, wl[e], lloc);
  }
  for (int o2 = 32; o2 >= 1; o2 >>= 1) lloc += __shfl_xor(lloc, o2);
  if ((c & 63) == 0) s_red[j][2 + (c >> 6)] = lloc;
  __syncthreads();
  const float l = s_red[j][2] + s_red[j][3];
  const float inv = l > 0.f ? 1.0f / l : 0.f;
  if (c == 0 && lse != nullptr) lse[(size_t)b * hq + jq] = l > 0.f ? M * kLn2 + logf(l) : -INFINITY;
  // o'[j][c] = sum_e w_e o'_e[c] / l over the INT2 slots in order, then the window slot; an
  // empty entry (w = 0) is skipped, so its partial output is never read into the sum.  Slots
  // past the first 16 are loaded 16 at a time.
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
  if (wj[ns - 1] > 0.f) acc = fmaf(wj[ns - 1], ow, acc);
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
    acc2 = fmaf(s_o[j][4 * k4 + 0], r.x, acc2);
    acc2 = fmaf(s_o[j][4 * k4 + 1], r.y, acc2);
    acc2 = fmaf(s_o[j][4 * k4 + 2], r.z, acc2);
    acc2 = fmaf(s_o[j][4 * k4 + 3], r.w, acc2);
  }
  orow[c] = acc2;
}

}  // namespace

hipError_t launch_combine(int batch, int hq, int hkv, const Workspace& ws, const float* rot_v,
                          float* out, float* lse, hipStream_t stream) {
  if (batch == 0) return hipSuccess;
  const size_t lds = (size_t)2 * (hq / hkv) * ws.nslots * sizeof(float);
  if (lds > 48 * 1024) return hipErrorInvalidValue;
  hipLaunchKernelGGL(combine_kernel, dim3(hkv, batch), dim3(128 * (hq / hkv)), lds, stream, hq, hkv,
                     ws, rot_v, out, lse);
  return hipGetLastError();
}

}  // namespace oscar
