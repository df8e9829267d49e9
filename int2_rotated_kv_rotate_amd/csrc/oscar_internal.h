// Internal definitions shared by the HIP translation units of the library.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace oscar {

constexpr int kHeadDim = 128;
constexpr int kPage = 16;
constexpr int kGroup = 32;
constexpr int kGroups = kHeadDim / kGroup;
constexpr int kRecord = 1536;                 // bytes per (page, KV head) INT2 record
constexpr int kKCodes = 0, kVCodes = 512, kKMeta = 1024, kVMeta = 1280;
constexpr int kBf16PageElems = 2 * kPage * kHeadDim;  // 4096 bf16 per (page, KV head)
constexpr int kMaxSinkWindow = 256;   // S + W
// The BF16 sink + window positions of a (sequence, KV head) pair are split into at most
// kWinSlots parts of kWinPartTokens positions (or kept whole), each with its own partial slot.
constexpr int kWinPartTokens = 32;
constexpr int kWinSlots = kMaxSinkWindow / kWinPartTokens;

// Workspace layout (all offsets in bytes from the workspace base).
//   Q region:  per (b, j) a 1024-byte block
//     [  0, 512) float q'[128]           rotated query (fp32)
//     [512, 640) int8  hi[128]           q' ~= qsc * (hi + lo/254), stored in MFMA slot order
//     [640, 768) int8  lo[128]
//     [768, 772) float qsc
//     [772, 788) float qsum[4]           sum of 254*hi + lo over each 32-channel group (exact)
//   O region:  float o'[B][Hq][nslots][128]   unnormalised partial outputs (rotated frame)
//   ML region: float2 (m, l)[B][Hq][nslots]  m in log2 units, l = sum of 2^(z*log2e - m)
//   Plan region (int32):
//     [0] total INT2 pages over all (sequence, KV head) pairs, [1] pages per worker run,
//     [2], [3] unused; then pstart[B] (first run index of sequence b's pairs: pair (b, h) owns
//     pages pstart[b] + h*npg[b] .. + npg[b] of the concatenation), npg[B] (INT2 pages per
//     KV head of sequence b), pglo[B] (first logical INT2 page of sequence b), and
//     nvalid[B][Hkv] (partial slots 0 .. nvalid-1 of the pair hold INT2 partials).
//   Slots 0 .. max_splits-1 of every (b, j) hold INT2 partials, the last kWinSlots slots
//   (max_splits .. nslots-1) the BF16 sink/window partials; a slot with l = 0 is empty.
constexpr int kQBlock = 1024;
constexpr int kQHiOff = 512, kQLoOff = 640, kQScOff = 768, kQSumOff = 772;
constexpr int kPlanHeader = 4;

struct Workspace {
  char* base;
  int batch;
  int nslots;  // max_splits + kWinSlots
  __host__ __device__ int max_splits() const { return nslots - kWinSlots; }
  __host__ __device__ int win_slot() const { return nslots - kWinSlots; }  // first window slot
  size_t q_bytes, o_bytes, ml_bytes, plan_bytes;
  __host__ __device__ char* qblock(int b, int hq, int j) const {
    return base + ((size_t)b * hq + j) * kQBlock;
  }
  __host__ __device__ float* o(int b, int hq, int j, int s) const {
    return (float*)(base + q_bytes) + (((size_t)b * hq + j) * nslots + s) * kHeadDim;
  }
  __host__ __device__ float2* ml(int b, int hq, int j, int s) const {
    return (float2*)(base + q_bytes + o_bytes) + ((size_t)b * hq + j) * nslots + s;
  }
  __host__ __device__ int32_t* plan() const {
    return (int32_t*)(base + q_bytes + o_bytes + ml_bytes);
  }
  __host__ __device__ int32_t* pstart() const { return plan() + kPlanHeader; }
  __host__ __device__ int32_t* npg() const { return pstart() + batch; }
  __host__ __device__ int32_t* pglo() const { return npg() + batch; }
  __host__ __device__ int32_t* nvalid() const { return pglo() + batch; }
};

// The plan sizes nvalid for Hq (>= Hkv) pairs per sequence so that its size needs no Hkv.
inline Workspace make_workspace(void* base, int batch, int hq, int max_splits) {
  Workspace w;
  w.base = (char*)base;
  w.batch = batch;
  w.nslots = max_splits + kWinSlots;
  w.q_bytes = (size_t)batch * hq * kQBlock;
  w.o_bytes = (size_t)batch * hq * w.nslots * kHeadDim * sizeof(float);
  w.ml_bytes = (size_t)batch * hq * w.nslots * sizeof(float2);
  w.plan_bytes = (((size_t)kPlanHeader + 3 * (size_t)batch + (size_t)batch * hq) * sizeof(int32_t) +
                  255) & ~(size_t)255;
  return w;
}

inline size_t workspace_bytes(int batch, int hq, int max_splits) {
  Workspace w = make_workspace(nullptr, batch, hq, max_splits);
  return w.q_bytes + w.o_bytes + w.ml_bytes + w.plan_bytes;
}

struct CacheGeom {
  int hkv, num_sink, window, num_pages, max_pages, num_slots;
};

// Host launchers (each defined next to its kernel).
// Append kernels (same bytes; speed differs): fp64 on the vector ALUs, or the matrix cores with
// certification and exact recomputation.  Auto takes the matrix cores from kMatrixAppendRows rows.
constexpr int kAppendAuto = 0, kAppendVector = 1, kAppendMatrix = 2;
constexpr int kMatrixAppendRows = 256;
hipError_t launch_append(const CacheGeom& g, uint8_t* pages, uint16_t* sinkwin,
                         const int32_t* block_table, const int32_t* slot_ids, int batch,
                         int total_new, const uint16_t* k_new, const uint16_t* v_new,
                         const int32_t* new_offsets, const int32_t* start_pos,
                         const float* rot_k, const float* rot_v, const float* k_mean,
                         float clip_k, float clip_v, int method, hipStream_t stream);

// Append with the Hadamard rotation diag(s) . H / sqrt(128) (fp64 fast transform); signs
// int8 [Hkv][128] (negative flips the input channel) or NULL for all +1.
hipError_t launch_append_hadamard(const CacheGeom& g, uint8_t* pages, uint16_t* sinkwin,
                                  const int32_t* block_table, const int32_t* slot_ids, int batch,
                                  int total_new, const uint16_t* k_new, const uint16_t* v_new,
                                  const int32_t* new_offsets, const int32_t* start_pos,
                                  const int8_t* signs_k, const int8_t* signs_v, float clip_k,
                                  float clip_v, hipStream_t stream);

// The q rotation and work plan (prep_q_kernel, step.hip) over `grid`: (Hkv * G / hpw, batch + 1)
// workgroups, hpw query heads each; the plan is built for `workers` INT2 workers.
hipError_t launch_prep_q_grid(dim3 grid, hipStream_t stream, const CacheGeom& g,
                              const uint16_t* q, const float* rot_k, int hq,
                              const int32_t* seq_lens, int workers, int hpw, const Workspace& ws);

// Worker count and query heads per preparation workgroup of the INT2 decode for this launch
// (decode.hip; the plan must be built for the decode kernel's own worker count).
void decode_prep_config(const CacheGeom& g, int batch, int hq, int num_workers, int* workers,
                        int* hpw);

// The new rows' append (as launch_append with kAppendAuto) and the INT2 decode's query
// preparation (as launch_decode_prep) in one launch when the append would take the 4-row vector
// kernel, else as the two launches (step.hip).  Same bytes as the two calls.
hipError_t launch_append_prepare(const CacheGeom& g, uint8_t* pages, uint16_t* sinkwin,
                                 const int32_t* block_table, const int32_t* slot_ids, int batch,
                                 int total_new, const uint16_t* k_new, const uint16_t* v_new,
                                 const int32_t* new_offsets, const int32_t* start_pos,
                                 const float* rot_k, const float* rot_v, const float* k_mean,
                                 float clip_k, float clip_v, int hq, const uint16_t* q,
                                 const int32_t* seq_lens, int num_workers, const Workspace& ws,
                                 hipStream_t stream);

hipError_t launch_decode(const CacheGeom& g, const uint8_t* pages, const uint16_t* sinkwin,
                         const int32_t* block_table, const int32_t* slot_ids, int batch,
                         int hq, const uint16_t* q, const int32_t* seq_lens, const float* rot_k,
                         float sm_scale, int num_workers, const Workspace& ws,
                         hipStream_t stream);

// q' = q . R_K (fp32 and int8 forms) into the workspace Q blocks, as oscar_decode_attention's
// first kernel does (its work plan is built for a single worker).
// The two halves of launch_decode: the q rotation and work plan, then the decode kernel (same
// batch, heads, lengths and num_workers; the workspace carries the q blocks and the plan).
hipError_t launch_decode_prep(const CacheGeom& g, const uint16_t* q, const float* rot_k, int batch,
                              int hq, const int32_t* seq_lens, int num_workers,
                              const Workspace& ws, hipStream_t stream);
hipError_t launch_decode_main(const CacheGeom& g, const uint8_t* pages, const uint16_t* sinkwin,
                              const int32_t* block_table, const int32_t* slot_ids, int batch,
                              int hq, const int32_t* seq_lens, float sm_scale, int num_workers,
                              const Workspace& ws, hipStream_t stream);

hipError_t launch_prep_q(const CacheGeom& g, const uint16_t* q, const float* rot_k, int batch,
                         int hq, const int32_t* seq_lens, const Workspace& ws, hipStream_t stream);

// INT4 cache (2560-byte records): append and decode (partials for launch_combine).
// The matrix-core prefill kernel for INT4 records (append.hip); launch_int4_append takes it from
// kMatrixAppendRows rows.
hipError_t launch_prefill_int4(const CacheGeom& g, uint8_t* pages, uint16_t* sinkwin,
                               const int32_t* block_table, const int32_t* slot_ids, int batch,
                               int total_new, const uint16_t* k_new, const uint16_t* v_new,
                               const int32_t* new_offsets, const int32_t* start_pos,
                               const float* rot_k, const float* rot_v, const float* k_mean,
                               float clip_k, float clip_v, hipStream_t stream);
hipError_t launch_int4_append(const CacheGeom& g, uint8_t* pages, uint16_t* sinkwin,
                              const int32_t* block_table, const int32_t* slot_ids, int batch,
                              int total_new, const uint16_t* k_new, const uint16_t* v_new,
                              const int32_t* new_offsets, const int32_t* start_pos,
                              const float* rot_k, const float* rot_v, const float* k_mean,
                              float clip_k, float clip_v, hipStream_t stream);
hipError_t launch_int4_decode(const CacheGeom& g, const uint8_t* pages, const uint16_t* sinkwin,
                              const int32_t* block_table, const int32_t* slot_ids, int batch,
                              int hq, const uint16_t* q, const int32_t* seq_lens,
                              const float* rot_k, float sm_scale, int split_pages,
                              const Workspace& ws, hipStream_t stream);

hipError_t launch_combine(int batch, int hq, int hkv, const Workspace& ws, const float* rot_v,
                          float* out, float* lse, hipStream_t stream);

// INT4 pages on the matrix cores (G <= 4): the INT2 launch shape with 2560-byte pages.
hipError_t launch_int4_mfma_decode(const CacheGeom& g, const uint8_t* pages,
                                  const uint16_t* sinkwin, const int32_t* block_table,
                                  const int32_t* slot_ids, int batch, int hq, const uint16_t* q,
                                  const int32_t* seq_lens, const float* rot_k, float sm_scale,
                                  const Workspace& ws, hipStream_t stream);

// Compute units of the current device, queried once per device and then read from a cache
// (launch paths call it on every launch); 0 when the query fails.
int current_device_cus();

// One bf16 matrix-core instruction per tile (D = A . B + C): see oscar_mfma_bf16_tiles.
hipError_t launch_mfma_bf16_tiles(const uint16_t* a, const uint16_t* b, const float* c, float* d,
                                  int tiles, hipStream_t stream);

// Read-bandwidth probe over INT2 records (no arithmetic): see oscar_read_records.
hipError_t launch_read_records(const uint8_t* pool, int num_records, const int32_t* record_ids,
                               int n, int workers, uint32_t* out, hipStream_t stream);

hipError_t launch_bf16_append(const CacheGeom& g, uint16_t* pages, const int32_t* block_table,
                              int batch, int total_new, const uint16_t* k_new,
                              const uint16_t* v_new, const int32_t* new_offsets,
                              const int32_t* start_pos, hipStream_t stream);

hipError_t launch_bf16_decode(const CacheGeom& g, const uint16_t* pages,
                              const int32_t* block_table, int batch, int hq, const uint16_t* q,
                              const int32_t* seq_lens, float sm_scale, int split_pages,
                              const Workspace& ws, hipStream_t stream);

// ---------------------------------------------------------------------------------- device

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float((uint32_t)b << 16);
}

// Round to nearest even (inputs are finite).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// The 32-bit value of lane (this lane ^ M): DPP within quads and rows where a pattern exists
// (M = 1, 2: quad permutes; M = 8: rotate a 16-lane row by 8), a swizzle within 32 lanes for
// M = 4, 16, and a lane permute for M = 32.
template <int M>
__device__ __forceinline__ uint32_t lane_xor(uint32_t v) {
  if constexpr (M == 1) return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, true);
  else if constexpr (M == 2) return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, true);
  else if constexpr (M == 8) return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x128, 0xF, 0xF, true);
  else if constexpr (M == 4 || M == 16) return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x1F | (M << 10));
  else return (uint32_t)__shfl_xor((int)v, M);
}
template <int M>
__device__ __forceinline__ double lane_xor_f64(double v) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = lane_xor<M>((uint32_t)u), hi = lane_xor<M>((uint32_t)(u >> 32));
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
template <int M>
__device__ __forceinline__ float lane_xor_f32(float v) {
  return __uint_as_float(lane_xor<M>(__float_as_uint(v)));
}
// Sequence index of flattened row n, given prefix offsets off[0..batch] (binary search).
__device__ __forceinline__ int row_to_seq(const int32_t* off, int batch, int n) {
  // find the largest b < batch with off[b] <= n.  First guess b = n (one new row per sequence,
  // as in decode): two independent loads settle it; otherwise bisect.
  const int g = min(n, batch - 1);
  const int og = off[g], og1 = off[g + 1];
  if (og <= n && (g == batch - 1 || og1 > n)) return g;
  int lo = 0, hi = batch;
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (off[mid] <= n) lo = mid; else hi = mid;
  }
  return lo;
}

// ------------------------------------------------------------- append helpers (INT2 and INT4)

// Keeps the compiler from fusing an fp32 result into a following conversion (it would
// otherwise turn fp16(c * mn) into one single-rounding mixed-precision FMA).
__device__ __forceinline__ float materialize(float x) {
  asm volatile("" : "+v"(x));
  return x;
}

struct RowInfo {
  long long rec;     // byte offset of the row's page record in the pool, -1 = skip
  int slot_in_page;  // 0..15
  long long sw;      // element offset of the row's bf16 K/V row in the store, -1 = none
};

// Where new row n (flattened over the batch) of KV head h goes, for records of REC bytes.
// The lookups take two rounds of dependent loads: the offsets, start position and store slot of
// the guessed sequence (b = n, one new row per sequence as in decode) together, then the block
// table entry; a wrong guess bisects the offsets.  row_lookup issues the first round, so that a
// caller can issue other loads before row_info_from waits for it.
struct RowLookup {
  int n, g, og, og1, sp, slot;
};
__device__ __forceinline__ RowLookup row_lookup(const int32_t* __restrict__ new_offsets,
                                                const int32_t* __restrict__ start_pos,
                                                const int32_t* __restrict__ slot_ids, int batch,
                                                int n) {
  RowLookup L;
  L.n = n;
  L.g = min(n, batch - 1);
  L.og = new_offsets[L.g];
  L.og1 = new_offsets[L.g + 1];
  L.sp = start_pos[L.g];
  L.slot = slot_ids ? slot_ids[L.g] : L.g;
  return L;
}

template <int REC>
__device__ RowInfo row_info_from(const CacheGeom& g, const int32_t* __restrict__ block_table,
                                 const int32_t* __restrict__ slot_ids, int batch,
                                 const int32_t* __restrict__ new_offsets,
                                 const int32_t* __restrict__ start_pos, bool has_store,
                                 const RowLookup& L, int h, bool is_v) {
  RowInfo info{-1, 0, -1};
  const int n = L.n;
  int b, first, nnew, sp, slot;
  if (L.og <= n && (L.g == batch - 1 || L.og1 > n)) {
    b = L.g;
    first = L.og;
    nnew = L.og1 - L.og;
    sp = L.sp;
    slot = L.slot;
  } else {
    b = row_to_seq(new_offsets, batch, n);
    first = new_offsets[b];
    nnew = new_offsets[b + 1] - first;
    sp = start_pos[b];
    slot = slot_ids ? slot_ids[b] : b;
  }
  const int pos = sp + (n - first);
  const int new_len = sp + nnew;
  const int lp = pos / kPage;
  if (pos >= 0 && lp < g.max_pages) {
    const int page = block_table[(size_t)b * g.max_pages + lp];
    if (page >= 0 && page < g.num_pages) {
      info.rec = ((long long)page * g.hkv + h) * REC;
      info.slot_in_page = pos % kPage;
    }
  }
  int row = -1;
  if (pos >= 0 && pos < g.num_sink) row = pos;
  else if (g.window > 0 && pos >= g.num_sink && pos >= new_len - g.window)
    row = g.num_sink + pos % g.window;
  if (row >= 0 && has_store && slot >= 0 && slot < g.num_slots)
    info.sw = (((long long)slot * g.hkv + h) * (g.num_sink + g.window) + row) * 2 * kHeadDim +
              (is_v ? kHeadDim : 0);
  return info;
}

template <int REC>
__device__ RowInfo row_info_t(const CacheGeom& g, const int32_t* __restrict__ block_table,
                              const int32_t* __restrict__ slot_ids, int batch,
                              const int32_t* __restrict__ new_offsets,
                              const int32_t* __restrict__ start_pos, bool has_store, int n, int h,
                              bool is_v) {
  return row_info_from<REC>(g, block_table, slot_ids, batch, new_offsets, start_pos, has_store,
                            row_lookup(new_offsets, start_pos, slot_ids, batch, n), h, is_v);
}

// fp16 scale and zero of a group from its extremes: s = (c*mx - c*mn) / STEPS, z = c*mn
// (STEPS = levels - 1), every step in fp32, a signed-zero extreme counting as +0.  Monotone: s
// never decreases with mx nor increases with mn, z never decreases with mn.
template <int STEPS>
__device__ __forceinline__ void group_params_t(float mx, float mn, float clip, _Float16& s16,
                                               _Float16& z16) {
  mx = mx + 0.0f;
  mn = mn + 0.0f;
  const float mx_c = clip * mx;
  const float mn_c = clip * mn;
  const float width = mx_c - mn_c;
  const float s32 = width / (float)STEPS;
  s16 = (_Float16)materialize(s32);
  z16 = (_Float16)materialize(mn_c);
}

// clamp(rint((y - z) / s), 0, STEPS), 0 for a zero scale.  Monotone in y for s > 0.
template <int STEPS>
__device__ __forceinline__ int code_of_t(float y, float s, float z) {
  if (s == 0.0f) return 0;
  float q = (y - z) / s;
  q = __builtin_rintf(q);
  q = fminf(fmaxf(q, 0.0f), (float)STEPS);
  return (int)q;
}

}  // namespace oscar
