// Split combine: merge the per-split softmax partials of each (sequence, query head) in a fixed
// ascending order, normalise, and rotate the output back with the transpose of the value
// rotation (o = o' . R_V^T, exact for orthogonal R_V; OSCAR paper, "Abstract": fixed rotations
// keep attention aligned with what it consumes).
//
// grid (Hkv, batch), block 128 (thread = output channel).  One workgroup serves the G query heads
// of a KV head, so each row of R_V is read once per workgroup.
#include "oscar_internal.h"

namespace oscar {
namespace {

constexpr float kLn2 = 0.69314718055994531f;

__global__ __launch_bounds__(128) void combine_kernel(int hq, int hkv, Workspace ws,
                                                     const float* __restrict__ rot_v,
                                                     float* __restrict__ out,
                                                     float* __restrict__ lse) {
  const int h = blockIdx.x, b = blockIdx.y, c = threadIdx.x;
  const int G = hq / hkv;
  __shared__ float s_o[8][kHeadDim];
  float inv_l[8];
  for (int j = 0; j < G; ++j) {
    const int jq = h * G + j;
    float M = -INFINITY;
    for (int s = 0; s < ws.nslots; ++s) {
      const float2 ml = *ws.ml(b, hq, jq, s);
      if (ml.y > 0.f) M = fmaxf(M, ml.x);
    }
    float l = 0.f, o = 0.f;
    for (int s = 0; s < ws.nslots; ++s) {
      const float2 ml = *ws.ml(b, hq, jq, s);
      if (ml.y > 0.f) {
        const float w = __builtin_amdgcn_exp2f(ml.x - M);
        l = fmaf(w, ml.y, l);
        o = fmaf(w, ws.o(b, hq, jq, s)[c], o);
      }
    }
    s_o[j][c] = l > 0.f ? o / l : 0.f;
    inv_l[j & 7] = l;
    if (c == 0 && lse != nullptr)
      lse[(size_t)b * hq + jq] = l > 0.f ? M * kLn2 + logf(l) : -INFINITY;
  }
  __syncthreads();
  (void)inv_l;
  float* orow = out + ((size_t)b * hq + h * G) * kHeadDim;
  if (rot_v == nullptr) {
    for (int j = 0; j < G; ++j) orow[j * kHeadDim + c] = s_o[j][c];
    return;
  }
  // out[j][c] = sum_k o'[j][k] * R_V[h][c][k]
  const float4* R = reinterpret_cast<const float4*>(rot_v + ((size_t)h * kHeadDim + c) * kHeadDim);
  float acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0.f;
  for (int k4 = 0; k4 < kHeadDim / 4; ++k4) {
    const float4 r = R[k4];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (j < G) {
        acc[j] = fmaf(s_o[j][4 * k4 + 0], r.x, acc[j]);
        acc[j] = fmaf(s_o[j][4 * k4 + 1], r.y, acc[j]);
        acc[j] = fmaf(s_o[j][4 * k4 + 2], r.z, acc[j]);
        acc[j] = fmaf(s_o[j][4 * k4 + 3], r.w, acc[j]);
      }
  }
#pragma unroll
  for (int j = 0; j < 8; ++j)
    if (j < G) orow[j * kHeadDim + c] = acc[j];
}

}  // namespace

hipError_t launch_combine(int batch, int hq, int hkv, const Workspace& ws, const float* rot_v,
                          float* out, float* lse, hipStream_t stream) {
  if (batch == 0) return hipSuccess;
  hipLaunchKernelGGL(combine_kernel, dim3(hkv, batch), dim3(128), 0, stream, hq, hkv, ws, rot_v,
                     out, lse);
  return hipGetLastError();
}

}  // namespace oscar
