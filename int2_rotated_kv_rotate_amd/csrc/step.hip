// One decode step's front half: the q rotation and work plan of the INT2 decode (prep_q_kernel,
// also launched on its own by the decode entry points), and one launch that runs the new
// tokens' rotate-clip-quantize-append beside it (append_prepare_kernel).  The two are
// independent (the append writes this step's K/V rows, the preparation reads q and the lengths),
// and each alone leaves most of the device idle, so one launch holds both sets of workgroups.
//
// Method: OSCAR project card "FutureMLS-Lab/OSCAR", section "How it works" (K/V rows rotated,
// clipped and stored in INT2 with BF16 sinks and window; attention in the rotated frame);
// OSCAR paper, "Abstract" (q rotated by the same fixed R_K, so q'.k' = q.k).
//
// Built without floating-point contraction, like the append (append_rows states it too), so the
// q encoding is the same code in both launches.
#include "oscar_internal.h"
#include "append_rows.h"

namespace oscar {
namespace {

// ------------------------------------------------------------------------ q rotation + plan

// One workgroup (256 threads) per (KV head, sequence): q' = q . R_K for the G query heads of
// the group (fp32), written to the workspace with its int8 form for the matrix cores:
// q' ~= qsc * (hi + lo / 254), hi/lo in [-127, 127], stored in MFMA slot order, plus the
// per-group sums of the encoded values.  Every global load is issued before its first use:
// R_K as 16 independent float4 loads per thread (partial sums over 16 input rows, reduced
// through LDS).  One more workgroup, (0, batch), builds the work plan of the INT2 kernel.
constexpr int kPrepThreads = 256;
static_assert(kPrepThreads == kAppendThreads, "one block size for both roles of the step launch");

constexpr int kPlanWaves = kPrepThreads / 64;

// Shared memory of one workgroup of prep_q_block (and build_plan).
struct PrepShared {
  int w[2][kPlanWaves];                                 // plan: per-wave sums, maxima, totals
  __attribute__((aligned(16))) float q[8][kHeadDim];    // q (bf16 widened)
  float qr[8][kHeadDim];                                // q' = q . R_K
  float4 part[8][8][kHeadDim / 4];                      // [input block][head][channel quad]
};

// Work plan for int2_decode_kernel, built by one workgroup (kPrepThreads threads).  The INT2
// pages of every (sequence, KV head) pair, laid end to end in (sequence, head) order, are cut
// into runs of C pages, one run per worker; C is the smallest length that needs at most
// `workers` runs and leaves no pair more than max_splits runs.
__device__ void build_plan(const CacheGeom& g, const int32_t* __restrict__ seq_lens, int workers,
                           const Workspace& ws, PrepShared& sm) {
  int (&s_w)[2][kPlanWaves] = sm.w;  // per-wave sums / maxima, then per-wave scan totals
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int B = ws.batch, max_splits = ws.max_splits();
  auto int2_pages = [&](int b, int& first) -> int {  // INT2 pages of sequence b, first page
    const int L = max(seq_lens[b], 0);
    const int n_sink = min(L, g.num_sink);
    const int lo = n_sink, hi = L - min(g.window, L - n_sink);
    first = lo / kPage;
    if (hi <= lo || g.num_pages < 1) return 0;
    return max(min((hi + kPage - 1) / kPage, g.max_pages) - first, 0);
  };
  // pass 1: total pages and the largest pair (wave reductions, then the waves in order)
  int tot = 0, pmax = 0;
  for (int b = t; b < B; b += kPrepThreads) {
    int first;
    const int P = int2_pages(b, first);
    tot += P * g.hkv;
    pmax = max(pmax, P);
  }
  for (int o = 32; o >= 1; o >>= 1) {
    tot += __shfl_xor(tot, o);
    pmax = max(pmax, __shfl_xor(pmax, o));
  }
  if (lane == 0) {
    s_w[0][wv] = tot;
    s_w[1][wv] = pmax;
  }
  __syncthreads();
  int total = 0;
  pmax = 0;
  for (int k = 0; k < kPlanWaves; ++k) {
    total += s_w[0][k];
    pmax = max(pmax, s_w[1][k]);
  }
  __syncthreads();
  long long C = max(1LL, ((long long)total + workers - 1) / workers);
  if (max_splits > 1) C = max(C, ((long long)pmax + max_splits - 2) / (max_splits - 1));
  else C = max(C, (long long)total);
  // pass 2: prefix sums in chunks of kPrepThreads sequences (a wave scan, then the waves'
  // totals in order), and the partial count of each (sequence, KV head) pair.  Page counts fit
  // in 31 bits (the plan stores them as int32), so the run arithmetic is unsigned 32-bit.
  int32_t* pstart = ws.pstart();
  int32_t* npg = ws.npg();
  int32_t* pglo = ws.pglo();
  int32_t* nvalid = ws.nvalid();
  const uint32_t Cu = (uint32_t)C;
  int carry = 0;
  for (int base = 0; base < B; base += kPrepThreads) {
    const int b = base + t;
    int first = 0;
    const int P = b < B ? int2_pages(b, first) : 0;
    const int x = P * g.hkv;
    int incl = x;
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o);
      if (lane >= o) incl += y;
    }
    if (lane == 63) s_w[0][wv] = incl;
    __syncthreads();
    int before = 0, chunk = 0;
    for (int k = 0; k < kPlanWaves; ++k) {
      before += k < wv ? s_w[0][k] : 0;
      chunk += s_w[0][k];
    }
    const int start = carry + before + incl - x;
    if (b < B) {
      pstart[b] = start;
      npg[b] = P;
      pglo[b] = first;
      const uint32_t Pp = (uint32_t)P;
      for (int h = 0; h < g.hkv; ++h) {
        const uint32_t s0 = (uint32_t)start + (uint32_t)h * Pp;
        nvalid[b * g.hkv + h] = Pp == 0 ? 0 : (int)((s0 + Pp - 1) / Cu - s0 / Cu + 1);
      }
    }
    carry += chunk;
    __syncthreads();
  }
  if (t == 0) {
    ws.plan()[0] = total;
    ws.plan()[1] = (int)C;
  }
}

// hpw: query heads per workgroup, G (one workgroup per KV head) or 1 (one per query head, for
// small batches: more workgroups, each with a quarter or less of the work).
// Workgroup (bx, by) of the query preparation: bx selects the KV head and its hpw query heads,
// by < ceil(batch / spb) the sequences spb*by .. spb*by + spb-1 (rows r = the sequence's index
// times hpw + the head's, spb * hpw <= 8, one R_K load for all); the extra row by ==
// ceil(batch / spb) builds the plan (bx == 0).  Each row's q' is computed the same way whatever
// spb and hpw are.
__device__ __forceinline__ void prep_q_block(
    const CacheGeom& g, const uint16_t* __restrict__ q, const float* __restrict__ rot_k, int hq,
    const int32_t* __restrict__ seq_lens, int workers, int hpw, int spb, const Workspace& ws,
    int bx, int by, PrepShared& sm) {
  const int t = threadIdx.x;
  if (by == (ws.batch + spb - 1) / spb) {  // the extra row of workgroups builds the plan
    if (bx == 0) build_plan(g, seq_lens, workers, ws, sm);
    return;
  }
  const int b0 = by * spb, nr = spb * hpw;
  const int lane = t & 63, wv = t >> 6;
  const int G = hq / g.hkv;
  const int h = bx / (G / hpw), j0 = (bx % (G / hpw)) * hpw;
  float (&s_q)[8][kHeadDim] = sm.q;
  float (&s_qr)[8][kHeadDim] = sm.qr;
  float4 (&s_part)[8][8][kHeadDim / 4] = sm.part;

  // Issue the R_K loads: thread -> channel quad c4 = t % 32, input block ib = t / 32 (16 rows).
  const int c4 = t & 31, ib = t >> 5;
  const float4* R4 = reinterpret_cast<const float4*>(rot_k + (size_t)h * kHeadDim * kHeadDim);
  float4 r[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) r[k] = R4[(16 * ib + k) * (kHeadDim / 4) + c4];
  for (int i = t; i < nr * kHeadDim; i += kPrepThreads) {
    const int rr = i / kHeadDim, c = i % kHeadDim, b = b0 + rr / hpw;
    s_q[rr][c] = b < ws.batch
                     ? bf16_to_f32(q[((size_t)b * hq + h * G + j0 + rr % hpw) * kHeadDim + c])
                     : 0.f;
  }
  __syncthreads();

  // q' partial sums over this thread's 16 input rows (ascending), one query head at a time,
  // its 16 q values read as four 16-byte loads; then reduce the 8 blocks in order.
  // (rows unrolled to the most a workgroup takes, so their independent chains interleave)
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (j >= nr) break;
    const float4* qp = reinterpret_cast<const float4*>(&s_q[j][16 * ib]);
    const float4 qv[4] = {qp[0], qp[1], qp[2], qp[3]};
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const float4& q4 = qv[k >> 2];
      const float qi = (k & 3) == 0 ? q4.x : (k & 3) == 1 ? q4.y : (k & 3) == 2 ? q4.z : q4.w;
      a.x = fmaf(qi, r[k].x, a.x);
      a.y = fmaf(qi, r[k].y, a.y);
      a.z = fmaf(qi, r[k].z, a.z);
      a.w = fmaf(qi, r[k].w, a.w);
    }
    s_part[ib][j][c4] = a;
  }
  __syncthreads();
  for (int e = t; e < nr * kHeadDim; e += kPrepThreads) {
    const int j = e / kHeadDim, c = e % kHeadDim;
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) s += reinterpret_cast<const float*>(&s_part[k][j][0])[c];
    s_qr[j][c] = s;
  }
  __syncthreads();

  // int8 form: wave wv handles rows wv, wv + 4; lane -> channels 2*lane, 2*lane + 1.
  for (int j = wv; j < nr; j += 4) {
    const int b = b0 + j / hpw;   // the same for the whole wave
    if (b >= ws.batch) continue;
    const float v0 = s_qr[j][2 * lane], v1 = s_qr[j][2 * lane + 1];
    // max |q'| over the wave: DPP within each row of 16 lanes, then the four rows' values
    float a = fmaxf(fabsf(v0), fabsf(v1));
    a = fmaxf(a, lane_xor_f32<1>(a));
    a = fmaxf(a, lane_xor_f32<2>(a));
    a = fmaxf(a, lane_xor_f32<4>(a));
    a = fmaxf(a, lane_xor_f32<8>(a));
    a = fmaxf(fmaxf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(a), 0)),
                    __int_as_float(__builtin_amdgcn_readlane(__float_as_int(a), 16))),
              fmaxf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(a), 32)),
                    __int_as_float(__builtin_amdgcn_readlane(__float_as_int(a), 48))));
    const float qsc = a / 127.0f;
    char* blk = ws.qblock(b, hq, h * G + j0 + j % hpw);
    int esum = 0;  // sum of the encoded values 254*hi + lo over this lane's two channels
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int c = 2 * lane + e;
      const float v = e ? v1 : v0;
      int hi = 0, lo = 0;
      if (qsc > 0.f) {
        hi = max(-127, min(127, (int)__builtin_rintf(v / qsc)));
        lo = max(-127, min(127, (int)__builtin_rintf((v - (float)hi * qsc) * 254.0f / qsc)));
      }
      esum += 254 * hi + lo;
      // slot order inside each 16-channel word: slot 4*i + b holds channel 4*b + i
      const int pos = 16 * (c / 16) + 4 * (c % 4) + (c % 16) / 4;
      blk[kQHiOff + pos] = (char)hi;
      blk[kQLoOff + pos] = (char)lo;
    }
    // The zero-point term of a logit uses these sums of the encoded q' (exact integers), so
    // that a key's code and zero parts see the same query: z*sum(q') and s*q'.codes then
    // carry one encoding error that cancels as in q'.k, instead of two that do not.
    esum += (int)lane_xor<1>((uint32_t)esum);   // the 16 lanes of a row = 32 channels
    esum += (int)lane_xor<2>((uint32_t)esum);
    esum += (int)lane_xor<4>((uint32_t)esum);
    esum += (int)lane_xor<8>((uint32_t)esum);
    reinterpret_cast<float2*>(blk)[lane] = make_float2(v0, v1);
    if (lane == 0) *reinterpret_cast<float*>(blk + kQScOff) = qsc;
    if ((lane & 15) == 0) reinterpret_cast<float*>(blk + kQSumOff)[lane >> 4] = (float)esum;
  }
}

__global__ __launch_bounds__(kPrepThreads) void prep_q_kernel(
    CacheGeom g, const uint16_t* __restrict__ q, const float* __restrict__ rot_k, int hq,
    const int32_t* __restrict__ seq_lens, int workers, int hpw, Workspace ws) {
  __shared__ PrepShared sm;
  prep_q_block(g, q, rot_k, hq, seq_lens, workers, hpw, 1, ws, blockIdx.x, blockIdx.y, sm);
}

// Append (4 rows per workgroup) and query preparation in one grid: workgroup 0 builds the
// plan, the next app_blocks are the append's (app_gx x Hkv x 2, x fastest), then the
// preparation's (prep_gx x ceil(batch / spb), x fastest).  The roles share one block of LDS.
union StepShared {
  AppendShared<4> a;
  PrepShared p;
};

__global__ __launch_bounds__(kPrepThreads) void append_prepare_kernel(
    CacheGeom g, uint8_t* __restrict__ pages, uint16_t* __restrict__ sinkwin,
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ slot_ids, int batch,
    int total_new, const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
    const int32_t* __restrict__ new_offsets, const int32_t* __restrict__ start_pos,
    const float* __restrict__ rot_k, const float* __restrict__ rot_v,
    const float* __restrict__ k_mean, float clip_k, float clip_v, const uint16_t* __restrict__ q,
    int hq, const int32_t* __restrict__ seq_lens, int workers, int hpw, int spb, Workspace ws,
    int app_blocks, int app_gx, int prep_gx) {
  __shared__ StepShared sm;
  const int id = blockIdx.x;
  if (id == 0) {  // the plan, first in the grid: its workgroup never waits for a free slot
    prep_q_block(g, q, rot_k, hq, seq_lens, workers, hpw, spb, ws, 0, (ws.batch + spb - 1) / spb,
                 sm.p);
  } else if (id - 1 < app_blocks) {
    const int a = id - 1, bx = a % app_gx, rest = a / app_gx;
    append_rows<4>(g, pages, sinkwin, block_table, slot_ids, batch, total_new, k_new, v_new,
                   new_offsets, start_pos, rot_k, rot_v, k_mean, clip_k, clip_v, bx,
                   rest % g.hkv, rest / g.hkv, sm.a);
  } else {
    const int p = id - 1 - app_blocks;
    prep_q_block(g, q, rot_k, hq, seq_lens, workers, hpw, spb, ws, p % prep_gx, p / prep_gx,
                 sm.p);
  }
}

}  // namespace

hipError_t launch_prep_q_grid(dim3 grid, hipStream_t stream, const CacheGeom& g,
                              const uint16_t* q, const float* rot_k, int hq,
                              const int32_t* seq_lens, int workers, int hpw, const Workspace& ws) {
  hipLaunchKernelGGL(prep_q_kernel, grid, dim3(kPrepThreads), 0, stream, g, q, rot_k, hq, seq_lens,
                     workers, hpw, ws);
  return hipGetLastError();
}

hipError_t launch_append_prepare(const CacheGeom& g, uint8_t* pages, uint16_t* sinkwin,
                                 const int32_t* block_table, const int32_t* slot_ids, int batch,
                                 int total_new, const uint16_t* k_new, const uint16_t* v_new,
                                 const int32_t* new_offsets, const int32_t* start_pos,
                                 const float* rot_k, const float* rot_v, const float* k_mean,
                                 float clip_k, float clip_v, int hq, const uint16_t* q,
                                 const int32_t* seq_lens, int num_workers, const Workspace& ws,
                                 hipStream_t stream) {
  if (batch == 0) return hipSuccess;
  int workers = 0, hpw = 0;
  decode_prep_config(g, batch, hq, num_workers, &workers, &hpw);
  const int prep_gx = g.hkv * (hq / g.hkv / hpw);
  // The append alone would take the vector kernel with 4 rows per workgroup below
  // kMatrixAppendRows rows; larger appends keep their own launch (same bytes either way).
  if (total_new == 0 || total_new >= kMatrixAppendRows) {
    if (total_new > 0) {
      const hipError_t e = launch_append(g, pages, sinkwin, block_table, slot_ids, batch,
                                         total_new, k_new, v_new, new_offsets, start_pos, rot_k,
                                         rot_v, k_mean, clip_k, clip_v, kAppendAuto, stream);
      if (e != hipSuccess) return e;
    }
    return launch_prep_q_grid(dim3(prep_gx, batch + 1), stream, g, q, rot_k, hq, seq_lens,
                              workers, hpw, ws);
  }
  // two sequences per preparation workgroup where its rows allow (one R_K load for both), so
  // that at two workgroups per CU (the append's LDS) the launch fits one round on more shapes
  const int spb = hpw <= 4 ? 2 : 1;
  const int app_gx = (total_new + 3) / 4;
  const int app_blocks = app_gx * g.hkv * 2;
  const long long blocks =
      (long long)app_blocks + (long long)prep_gx * ((batch + spb - 1) / spb) + 1;
  hipLaunchKernelGGL(append_prepare_kernel, dim3((unsigned)blocks), dim3(kPrepThreads), 0, stream,
                     g, pages, sinkwin, block_table, slot_ids, batch, total_new, k_new, v_new,
                     new_offsets, start_pos, rot_k, rot_v, k_mean, clip_k, clip_v, q, hq, seq_lens,
                     workers, hpw, spb, ws, app_blocks, app_gx, prep_gx);
  return hipGetLastError();
}

}  // namespace oscar
