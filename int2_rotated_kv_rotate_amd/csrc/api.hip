// C ABI entry points: validate host-visible arguments, then enqueue the kernels on the caller's
// stream.  No allocation and no synchronisation; the only state is a per-device cache of the
// compute-unit count and of the static workspace address.
#include <atomic>
#include <mutex>

#include "../../include/oscar.h"
#include "oscar_internal.h"

using namespace oscar;

namespace {

int32_t check_layout(const oscar_layout* lay) {
  if (lay == nullptr) return OSCAR_ERR_INVALID_ARGUMENT;
  if (lay->head_dim != kHeadDim || lay->page_size != kPage || lay->group_size != kGroup)
    return OSCAR_ERR_UNSUPPORTED;
  if (lay->num_kv_heads < 1 || lay->num_kv_heads > 65535) return OSCAR_ERR_INVALID_ARGUMENT;
  if (lay->num_sink < 0 || lay->window < 0) return OSCAR_ERR_INVALID_ARGUMENT;
  if ((long long)lay->num_sink + lay->window > kMaxSinkWindow) return OSCAR_ERR_UNSUPPORTED;
  if (lay->num_pages < 0 || lay->max_pages_per_seq < 1 || lay->num_slots < 0)
    return OSCAR_ERR_INVALID_ARGUMENT;
  return OSCAR_OK;
}

CacheGeom geom(const oscar_layout* lay) {
  return CacheGeom{lay->num_kv_heads, lay->num_sink, lay->window,
                   lay->num_pages, lay->max_pages_per_seq, lay->num_slots};
}

int32_t check_heads(int32_t hq, int32_t hkv) {
  if (hq < 1 || hq % hkv != 0) return OSCAR_ERR_INVALID_ARGUMENT;
  const int G = hq / hkv;
  if (G != 1 && G != 2 && G != 4 && G != 8) return OSCAR_ERR_UNSUPPORTED;
  return OSCAR_OK;
}

// Slots per (sequence, query head): 2 * G * (max_splits + kWinSlots) floats fit 48 KiB (a limit
// of the C ABI; the per-query-head combine keeps one float per slot in LDS).
int32_t check_splits(int32_t hq, int32_t hkv, int32_t max_splits) {
  if (max_splits < 1) return OSCAR_ERR_INVALID_ARGUMENT;
  if ((size_t)2 * (hq / hkv) * ((size_t)max_splits + kWinSlots) * sizeof(float) > 48 * 1024)
    return OSCAR_ERR_UNSUPPORTED;
  return OSCAR_OK;
}

constexpr int32_t kMaxWorkers = 1 << 20;

// batch * num_q_heads rows of queries, partials and outputs: at most 2^27, so that every grid
// size and index the launchers derive from them fits in int32 and the workspace size cannot
// wrap in size_t.
constexpr long long kMaxQueryRows = 1LL << 27;
int32_t check_rows(int32_t batch, int32_t hq) {
  return (long long)batch * hq > kMaxQueryRows ? OSCAR_ERR_UNSUPPORTED : OSCAR_OK;
}

// New rows of one append call: at most 2^30 (the launchers round the count up to tiles in int32).
constexpr int32_t kMaxNewRows = 1 << 30;

int32_t hip_status(hipError_t e) { return e == hipSuccess ? OSCAR_OK : OSCAR_ERR_HIP; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// A softmax scale must be finite and positive: the INT2 workers fold it into a strictly
// positive logit scale, while the BF16 sink/window logits use it as given.
bool valid_scale(float s) { return s > 0.f && s <= 3.402823466e38f; }

// Decode workspace for oscar_decode_attention_static: one copy per GPU, in device memory for
// the life of the process.  Host code never passes the array's name to a kernel (on the host
// it is only a stand-in for the symbol): it looks up the device address of this device's copy
// once and uses that address everywhere.
constexpr size_t kStaticWorkspaceBytes = OSCAR_STATIC_WORKSPACE_BYTES;
__device__ __attribute__((aligned(256))) unsigned char scratch[kStaticWorkspaceBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];   // device address of `scratch` per device, set once

// Device address of the current device's `scratch` (looked up on the first call per device).
hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr || ((uintptr_t)p & 255u) != 0) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

int oscar::current_device_cus() {
  static std::atomic<int> cus[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
  int n = cus[dev].load(std::memory_order_relaxed);
  if (n > 0) return n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    return 0;
  cus[dev].store(n, std::memory_order_relaxed);
  return n;
}

extern "C" {

const char* oscar_status_string(int32_t status) {
  switch (status) {
    case OSCAR_OK: return "ok";
    case OSCAR_ERR_INVALID_ARGUMENT: return "invalid argument";
    case OSCAR_ERR_UNSUPPORTED: return "unsupported geometry";
    case OSCAR_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case OSCAR_ERR_HIP: return "HIP launch failure";
    default: return "unknown status";
  }
}

int32_t oscar_rotate_quantize_append_ex(
    const oscar_layout* lay, uint8_t* pages, uint16_t* sinkwin,
    const int32_t* block_table, const int32_t* slot_ids,
    int32_t batch, int32_t total_new,
    const uint16_t* k_new, const uint16_t* v_new,
    const int32_t* new_offsets, const int32_t* start_pos,
    const float* rot_k, const float* rot_v, const float* k_mean, float clip_k, float clip_v,
    int32_t method, void* stream) {
  int32_t st = check_layout(lay);
  if (st != OSCAR_OK) return st;
  if (batch < 0 || total_new < 0) return OSCAR_ERR_INVALID_ARGUMENT;
  if (total_new > kMaxNewRows) return OSCAR_ERR_UNSUPPORTED;
  if (method != OSCAR_APPEND_AUTO && method != OSCAR_APPEND_VECTOR && method != OSCAR_APPEND_MATRIX)
    return OSCAR_ERR_INVALID_ARGUMENT;
  if (!(clip_k > 0.f && clip_k <= 1.f) || !(clip_v > 0.f && clip_v <= 1.f))
    return OSCAR_ERR_INVALID_ARGUMENT;
  if (batch == 0 || total_new == 0) return OSCAR_OK;
  if (!pages || !block_table || !k_new || !v_new || !new_offsets || !start_pos || !rot_k || !rot_v)
    return OSCAR_ERR_INVALID_ARGUMENT;
  if (lay->num_sink + lay->window > 0 && sinkwin == nullptr) return OSCAR_ERR_INVALID_ARGUMENT;
  if (!aligned16(pages) || !aligned16(k_new) || !aligned16(v_new) || !aligned16(rot_k) ||
      !aligned16(rot_v) || (sinkwin && !aligned16(sinkwin)) || ((uintptr_t)k_mean & 3u) != 0)
    return OSCAR_ERR_INVALID_ARGUMENT;
  static_assert(OSCAR_APPEND_AUTO == kAppendAuto && OSCAR_APPEND_VECTOR == kAppendVector &&
                OSCAR_APPEND_MATRIX == kAppendMatrix, "append method numbering");
  return hip_status(launch_append(geom(lay), pages, sinkwin, block_table, slot_ids, batch,
                                  total_new, k_new, v_new, new_offsets, start_pos, rot_k, rot_v,
                                  k_mean, clip_k, clip_v, method, (hipStream_t)stream));
}

int32_t oscar_rotate_quantize_append(
    const oscar_layout* lay, uint8_t* pages, uint16_t* sinkwin,
    const int32_t* block_table, const int32_t* slot_ids,
    int32_t batch, int32_t total_new,
    const uint16_t* k_new, const uint16_t* v_new,
    const int32_t* new_offsets, const int32_t* start_pos,
    const float* rot_k, const float* rot_v, float clip_k, float clip_v,
    void* stream) {
  return oscar_rotate_quantize_append_ex(lay, pages, sinkwin, block_table, slot_ids, batch,
                                         total_new, k_new, v_new, new_offsets, start_pos, rot_k,
                                         rot_v, nullptr, clip_k, clip_v, OSCAR_APPEND_AUTO, stream);
}

int32_t oscar_rotate_quantize_append_hadamard(
    const oscar_layout* lay, uint8_t* pages, uint16_t* sinkwin,
    const int32_t* block_table, const int32_t* slot_ids,
    int32_t batch, int32_t total_new,
    const uint16_t* k_new, const uint16_t* v_new,
    const int32_t* new_offsets, const int32_t* start_pos,
    const int8_t* signs_k, const int8_t* signs_v, float clip_k, float clip_v,
    void* stream) {
  int32_t st = check_layout(lay);
  if (st != OSCAR_OK) return st;
  if (batch < 0 || total_new < 0) return OSCAR_ERR_INVALID_ARGUMENT;
  if (total_new > kMaxNewRows) return OSCAR_ERR_UNSUPPORTED;
  if (!(clip_k > 0.f && clip_k <= 1.f) || !(clip_v > 0.f && clip_v <= 1.f))
    return OSCAR_ERR_INVALID_ARGUMENT;
  if (batch == 0 || total_new == 0) return OSCAR_OK;
  if (!pages || !block_table || !k_new || !v_new || !new_offsets || !start_pos)
    return OSCAR_ERR_INVALID_ARGUMENT;
  if (lay->num_sink + lay->window > 0 && sinkwin == nullptr) return OSCAR_ERR_INVALID_ARGUMENT;
  if (!aligned16(pages) || !aligned16(k_new) || !aligned16(v_new) || (sinkwin && !aligned16(sinkwin)))
    return OSCAR_ERR_INVALID_ARGUMENT;
  return hip_status(launch_append_hadamard(geom(lay), pages, sinkwin, block_table, slot_ids, batch,
                                           total_new, k_new, v_new, new_offsets, start_pos,
                                           signs_k, signs_v, clip_k, clip_v, (hipStream_t)stream));
}

int32_t oscar_int4_rotate_quantize_append(
    const oscar_layout* lay, uint8_t* pages, uint16_t* sinkwin,
    const int32_t* block_table, const int32_t* slot_ids,
    int32_t batch, int32_t total_new,
    const uint16_t* k_new, const uint16_t* v_new,
    const int32_t* new_offsets, const int32_t* start_pos,
    const float* rot_k, const float* rot_v, const float* k_mean, float clip_k, float clip_v,
    void* stream) {
  int32_t st = check_layout(lay);
  if (st != OSCAR_OK) return st;
  if (batch < 0 || total_new < 0) return OSCAR_ERR_INVALID_ARGUMENT;
  if (total_new > kMaxNewRows) return OSCAR_ERR_UNSUPPORTED;
  if (!(clip_k > 0.f && clip_k <= 1.f) || !(clip_v > 0.f && clip_v <= 1.f))
    return OSCAR_ERR_INVALID_ARGUMENT;
  if (batch == 0 || total_new == 0) return OSCAR_OK;
  if (!pages || !block_table || !k_new || !v_new || !new_offsets || !start_pos || !rot_k || !rot_v)
    return OSCAR_ERR_INVALID_ARGUMENT;
  if (lay->num_sink + lay->window > 0 && sinkwin == nullptr) return OSCAR_ERR_INVALID_ARGUMENT;
  if (!aligned16(pages) || !aligned16(k_new) || !aligned16(v_new) || !aligned16(rot_k) ||
      !aligned16(rot_v) || (sinkwin && !aligned16(sinkwin)) || ((uintptr_t)k_mean & 3u) != 0)
    return OSCAR_ERR_INVALID_ARGUMENT;
  return hip_status(launch_int4_append(geom(lay), pages, sinkwin, block_table, slot_ids, batch,
                                       total_new, k_new, v_new, new_offsets, start_pos, rot_k,
                                       rot_v, k_mean, clip_k, clip_v, (hipStream_t)stream));
}

int32_t oscar_int4_decode_attention(
    const oscar_layout* lay, const uint8_t* pages, const uint16_t* sinkwin,
    const int32_t* block_table, const int32_t* slot_ids,
    int32_t batch, int32_t num_q_heads,
    const uint16_t* q, const int32_t* seq_lens, const float* rot_k, float sm_scale,
    int32_t split_pages, int32_t max_splits,
    void* workspace, size_t workspace_bytes_given, void* stream) {
  int32_t st = check_layout(lay);
  if (st != OSCAR_OK) return st;
  if (batch < 0 || split_pages < 1 || max_splits < 1 || max_splits > 65535)
    return OSCAR_ERR_INVALID_ARGUMENT;
  st = check_heads(num_q_heads, lay->num_kv_heads);
  if (st != OSCAR_OK) return st;
  st = check_rows(batch, num_q_heads);
  if (st != OSCAR_OK) return st;
  st = check_splits(num_q_heads, lay->num_kv_heads, max_splits);
  if (st != OSCAR_OK) return st;
  if (!valid_scale(sm_scale)) return OSCAR_ERR_INVALID_ARGUMENT;
  if (batch == 0) return OSCAR_OK;
  if (!pages || !block_table || !q || !seq_lens || !rot_k || !workspace)
    return OSCAR_ERR_INVALID_ARGUMENT;
  if (lay->num_sink + lay->window > 0 && sinkwin == nullptr) return OSCAR_ERR_INVALID_ARGUMENT;
  if (!aligned16(pages) || !aligned16(q) || !aligned16(workspace) || !aligned16(rot_k) ||
      (sinkwin && !aligned16(sinkwin)))
    return OSCAR_ERR_INVALID_ARGUMENT;
  if (workspace_bytes_given < workspace_bytes(batch, num_q_heads, max_splits))
    return OSCAR_ERR_WORKSPACE_TOO_SMALL;
  Workspace ws = make_workspace(workspace, batch, num_q_heads, max_splits);
  return hip_status(launch_int4_decode(geom(lay), pages, sinkwin, block_table, slot_ids, batch,
                                       num_q_heads, q, seq_lens, rot_k, sm_scale, split_pages, ws,
                                       (hipStream_t)stream));
}

size_t oscar_decode_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t max_splits) {
  if (batch < 0 || num_q_heads < 1 || max_splits < 1 || max_splits > 65535) return 0;
  if (check_rows(batch, num_q_heads) != OSCAR_OK) return 0;
  return workspace_bytes(batch, num_q_heads, max_splits);
}

int32_t oscar_decode_attention(
    const oscar_layout* lay, const uint8_t* pages, const uint16_t* sinkwin,
    const int32_t* block_table, const int32_t* slot_ids,
    int32_t batch, int32_t num_q_heads,
    const uint16_t* q, const int32_t* seq_lens, const float* rot_k, float sm_scale,
    int32_t num_workers, int32_t max_splits,
    void* workspace, size_t workspace_bytes_given, void* stream) {
  int32_t st = check_layout(lay);
  if (st != OSCAR_OK) return st;
  if (batch < 0 || num_workers < 0 || num_workers > kMaxWorkers || max_splits < 1 ||
      max_splits > 65535)
    return OSCAR_ERR_INVALID_ARGUMENT;
  // page counts of the work plan are int32
  if ((long long)batch * lay->num_kv_heads * lay->max_pages_per_seq > 0x7FFFFFFFLL)
    return OSCAR_ERR_UNSUPPORTED;
  st = check_heads(num_q_heads, lay->num_kv_heads);
  if (st != OSCAR_OK) return st;
  st = check_rows(batch, num_q_heads);
  if (st != OSCAR_OK) return st;
  st = check_splits(num_q_heads, lay->num_kv_heads, max_splits);
  if (st != OSCAR_OK) return st;
  if (!valid_scale(sm_scale)) return OSCAR_ERR_INVALID_ARGUMENT;
  if (batch == 0) return OSCAR_OK;
  if (!pages || !block_table || !q || !seq_lens || !rot_k || !workspace)
    return OSCAR_ERR_INVALID_ARGUMENT;
  if (lay->num_sink + lay->window > 0 && sinkwin == nullptr) return OSCAR_ERR_INVALID_ARGUMENT;
  if (!aligned16(pages) || !aligned16(q) || !aligned16(workspace) || !aligned16(rot_k) ||
      (sinkwin && !aligned16(sinkwin)))
    return OSCAR_ERR_INVALID_ARGUMENT;
  if (workspace_bytes_given < workspace_bytes(batch, num_q_heads, max_splits))
    return OSCAR_ERR_WORKSPACE_TOO_SMALL;
  Workspace ws = make_workspace(workspace, batch, num_q_heads, max_splits);
  return hip_status(launch_decode(geom(lay), pages, sinkwin, block_table, slot_ids, batch,
                                  num_q_heads, q, seq_lens, rot_k, sm_scale, num_workers, ws,
                                  (hipStream_t)stream));
}

// Checks shared by the two halves of oscar_decode_attention (everything that does not concern
// one half's own pointers).
int32_t check_decode_common(const oscar_layout* lay, int32_t batch, int32_t num_q_heads,
                            int32_t num_workers, int32_t max_splits) {
  int32_t st = check_layout(lay);
  if (st != OSCAR_OK) return st;
  if (batch < 0 || num_workers < 0 || num_workers > kMaxWorkers || max_splits < 1 ||
      max_splits > 65535)
    return OSCAR_ERR_INVALID_ARGUMENT;
  if ((long long)batch * lay->num_kv_heads * lay->max_pages_per_seq > 0x7FFFFFFFLL)
    return OSCAR_ERR_UNSUPPORTED;
  st = check_heads(num_q_heads, lay->num_kv_heads);
  if (st != OSCAR_OK) return st;
  st = check_rows(batch, num_q_heads);
  if (st != OSCAR_OK) return st;
  return check_splits(num_q_heads, lay->num_kv_heads, max_splits);
}

int32_t oscar_prepare_queries(const oscar_layout* lay, int32_t batch, int32_t num_q_heads,
                              const uint16_t* q, const int32_t* seq_lens, const float* rot_k,
                              int32_t num_workers, int32_t max_splits, void* workspace,
                              size_t workspace_bytes_given, void* stream) {
  const int32_t st = check_decode_common(lay, batch, num_q_heads, num_workers, max_splits);
  if (st != OSCAR_OK) return st;
  if (batch == 0) return OSCAR_OK;
  if (!q || !seq_lens || !rot_k || !workspace) return OSCAR_ERR_INVALID_ARGUMENT;
  if (!aligned16(q) || !aligned16(workspace) || !aligned16(rot_k)) return OSCAR_ERR_INVALID_ARGUMENT;
  if (workspace_bytes_given < workspace_bytes(batch, num_q_heads, max_splits))
    return OSCAR_ERR_WORKSPACE_TOO_SMALL;
  Workspace ws = make_workspace(workspace, batch, num_q_heads, max_splits);
  return hip_status(launch_decode_prep(geom(lay), q, rot_k, batch, num_q_heads, seq_lens,
                                       num_workers, ws, (hipStream_t)stream));
}

int32_t oscar_append_and_prepare(
    const oscar_layout* lay, uint8_t* pages, uint16_t* sinkwin, const int32_t* block_table,
    const int32_t* slot_ids, int32_t batch, int32_t total_new, const uint16_t* k_new,
    const uint16_t* v_new, const int32_t* new_offsets, const int32_t* start_pos,
    const float* rot_k, const float* rot_v, const float* k_mean, float clip_k, float clip_v,
    int32_t num_q_heads, const uint16_t* q, const int32_t* seq_lens, int32_t num_workers,
    int32_t max_splits, void* workspace, size_t workspace_bytes_given, void* stream) {
  int32_t st = check_decode_common(lay, batch, num_q_heads, num_workers, max_splits);
  if (st != OSCAR_OK) return st;
  if (total_new < 0) return OSCAR_ERR_INVALID_ARGUMENT;
  if (total_new > kMaxNewRows) return OSCAR_ERR_UNSUPPORTED;
  if (!(clip_k > 0.f && clip_k <= 1.f) || !(clip_v > 0.f && clip_v <= 1.f))
    return OSCAR_ERR_INVALID_ARGUMENT;
  if (batch == 0) return OSCAR_OK;
  // the query preparation's arguments
  if (!q || !seq_lens || !rot_k || !workspace) return OSCAR_ERR_INVALID_ARGUMENT;
  if (!aligned16(q) || !aligned16(workspace) || !aligned16(rot_k)) return OSCAR_ERR_INVALID_ARGUMENT;
  if (workspace_bytes_given < workspace_bytes(batch, num_q_heads, max_splits))
    return OSCAR_ERR_WORKSPACE_TOO_SMALL;
  // the append's (none when there are no new rows)
  if (total_new > 0) {
    if (!pages || !block_table || !k_new || !v_new || !new_offsets || !start_pos || !rot_v)
      return OSCAR_ERR_INVALID_ARGUMENT;
    if (lay->num_sink + lay->window > 0 && sinkwin == nullptr) return OSCAR_ERR_INVALID_ARGUMENT;
    if (!aligned16(pages) || !aligned16(k_new) || !aligned16(v_new) || !aligned16(rot_v) ||
        (sinkwin && !aligned16(sinkwin)) || ((uintptr_t)k_mean & 3u) != 0)
      return OSCAR_ERR_INVALID_ARGUMENT;
  }
  Workspace ws = make_workspace(workspace, batch, num_q_heads, max_splits);
  return hip_status(launch_append_prepare(geom(lay), pages, sinkwin, block_table, slot_ids, batch,
                                          total_new, k_new, v_new, new_offsets, start_pos, rot_k,
                                          rot_v, k_mean, clip_k, clip_v, num_q_heads, q, seq_lens,
                                          num_workers, ws, (hipStream_t)stream));
}

int32_t oscar_decode_attention_prepared(
    const oscar_layout* lay, const uint8_t* pages, const uint16_t* sinkwin,
    const int32_t* block_table, const int32_t* slot_ids, int32_t batch, int32_t num_q_heads,
    const int32_t* seq_lens, float sm_scale, int32_t num_workers, int32_t max_splits,
    void* workspace, size_t workspace_bytes_given, void* stream) {
  const int32_t st = check_decode_common(lay, batch, num_q_heads, num_workers, max_splits);
  if (st != OSCAR_OK) return st;
  if (!valid_scale(sm_scale)) return OSCAR_ERR_INVALID_ARGUMENT;
  if (batch == 0) return OSCAR_OK;
  if (!pages || !block_table || !seq_lens || !workspace) return OSCAR_ERR_INVALID_ARGUMENT;
  if (lay->num_sink + lay->window > 0 && sinkwin == nullptr) return OSCAR_ERR_INVALID_ARGUMENT;
  if (!aligned16(pages) || !aligned16(workspace) || (sinkwin && !aligned16(sinkwin)))
    return OSCAR_ERR_INVALID_ARGUMENT;
  if (workspace_bytes_given < workspace_bytes(batch, num_q_heads, max_splits))
    return OSCAR_ERR_WORKSPACE_TOO_SMALL;
  Workspace ws = make_workspace(workspace, batch, num_q_heads, max_splits);
  return hip_status(launch_decode_main(geom(lay), pages, sinkwin, block_table, slot_ids, batch,
                                       num_q_heads, seq_lens, sm_scale, num_workers, ws,
                                       (hipStream_t)stream));
}

int32_t oscar_decode_attention_static(
    const oscar_layout* lay, const uint8_t* pages, const uint16_t* sinkwin,
    const int32_t* block_table, const int32_t* slot_ids,
    int32_t batch, int32_t num_q_heads,
    const uint16_t* q, const int32_t* seq_lens, const float* rot_k, const float* rot_v,
    float sm_scale, int32_t num_workers, int32_t max_splits,
    float* out, float* lse, void* stream) {
  int32_t st = check_layout(lay);
  if (st != OSCAR_OK) return st;
  if (batch < 0 || num_workers < 0 || num_workers > kMaxWorkers || max_splits < 1 ||
      max_splits > 65535)
    return OSCAR_ERR_INVALID_ARGUMENT;
  if ((long long)batch * lay->num_kv_heads * lay->max_pages_per_seq > 0x7FFFFFFFLL)
    return OSCAR_ERR_UNSUPPORTED;
  st = check_heads(num_q_heads, lay->num_kv_heads);
  if (st != OSCAR_OK) return st;
  st = check_rows(batch, num_q_heads);
  if (st != OSCAR_OK) return st;
  st = check_splits(num_q_heads, lay->num_kv_heads, max_splits);
  if (st != OSCAR_OK) return st;
  if (!valid_scale(sm_scale)) return OSCAR_ERR_INVALID_ARGUMENT;
  if (batch == 0) return OSCAR_OK;
  if (!pages || !block_table || !q || !seq_lens || !rot_k || !out)
    return OSCAR_ERR_INVALID_ARGUMENT;
  if (lay->num_sink + lay->window > 0 && sinkwin == nullptr) return OSCAR_ERR_INVALID_ARGUMENT;
  if (!aligned16(pages) || !aligned16(q) || !aligned16(rot_k) || (rot_v && !aligned16(rot_v)) ||
      (sinkwin && !aligned16(sinkwin)))
    return OSCAR_ERR_INVALID_ARGUMENT;
  if (workspace_bytes(batch, num_q_heads, max_splits) > kStaticWorkspaceBytes)
    return OSCAR_ERR_WORKSPACE_TOO_SMALL;
  void* base = nullptr;
  if (scratch_address(&base) != hipSuccess) return OSCAR_ERR_HIP;
  Workspace ws = make_workspace(base, batch, num_q_heads, max_splits);
  const hipStream_t s = (hipStream_t)stream;
  st = hip_status(launch_decode(geom(lay), pages, sinkwin, block_table, slot_ids, batch,
                                num_q_heads, q, seq_lens, rot_k, sm_scale, num_workers, ws, s));
  if (st != OSCAR_OK) return st;
  return hip_status(launch_combine(batch, num_q_heads, lay->num_kv_heads, ws, rot_v, out, lse, s));
}

int32_t oscar_combine(
    int32_t batch, int32_t num_q_heads, int32_t num_kv_heads, int32_t max_splits,
    const void* workspace, size_t workspace_bytes_given, const float* rot_v,
    float* out, float* lse, void* stream) {
  if (batch < 0 || num_kv_heads < 1 || max_splits < 1 || max_splits > 65535)
    return OSCAR_ERR_INVALID_ARGUMENT;
  int32_t st = check_heads(num_q_heads, num_kv_heads);
  if (st != OSCAR_OK) return st;
  st = check_rows(batch, num_q_heads);
  if (st != OSCAR_OK) return st;
  st = check_splits(num_q_heads, num_kv_heads, max_splits);
  if (st != OSCAR_OK) return st;
  if (batch == 0) return OSCAR_OK;
  if (!workspace || !out) return OSCAR_ERR_INVALID_ARGUMENT;
  if (!aligned16(workspace) || (rot_v && !aligned16(rot_v))) return OSCAR_ERR_INVALID_ARGUMENT;
  if (workspace_bytes_given < workspace_bytes(batch, num_q_heads, max_splits))
    return OSCAR_ERR_WORKSPACE_TOO_SMALL;
  Workspace ws = make_workspace(const_cast<void*>(workspace), batch, num_q_heads, max_splits);
  return hip_status(launch_combine(batch, num_q_heads, num_kv_heads, ws, rot_v, out, lse,
                                   (hipStream_t)stream));
}

int32_t oscar_bf16_append(
    const oscar_layout* lay, uint16_t* pages, const int32_t* block_table,
    int32_t batch, int32_t total_new, const uint16_t* k_new, const uint16_t* v_new,
    const int32_t* new_offsets, const int32_t* start_pos, void* stream) {
  int32_t st = check_layout(lay);
  if (st != OSCAR_OK) return st;
  if (batch < 0 || total_new < 0) return OSCAR_ERR_INVALID_ARGUMENT;
  if (total_new > kMaxNewRows) return OSCAR_ERR_UNSUPPORTED;
  if (batch == 0 || total_new == 0) return OSCAR_OK;
  if (!pages || !block_table || !k_new || !v_new || !new_offsets || !start_pos)
    return OSCAR_ERR_INVALID_ARGUMENT;
  if (!aligned16(pages) || !aligned16(k_new) || !aligned16(v_new)) return OSCAR_ERR_INVALID_ARGUMENT;
  return hip_status(launch_bf16_append(geom(lay), pages, block_table, batch, total_new, k_new,
                                       v_new, new_offsets, start_pos, (hipStream_t)stream));
}

int32_t oscar_bf16_decode_attention(
    const oscar_layout* lay, const uint16_t* pages, const int32_t* block_table,
    int32_t batch, int32_t num_q_heads, const uint16_t* q, const int32_t* seq_lens,
    float sm_scale, int32_t split_pages, int32_t max_splits,
    void* workspace, size_t workspace_bytes_given, void* stream) {
  int32_t st = check_layout(lay);
  if (st != OSCAR_OK) return st;
  if (batch < 0 || split_pages < 1 || max_splits < 1 || max_splits > 65535)
    return OSCAR_ERR_INVALID_ARGUMENT;
  st = check_heads(num_q_heads, lay->num_kv_heads);
  if (st != OSCAR_OK) return st;
  st = check_rows(batch, num_q_heads);
  if (st != OSCAR_OK) return st;
  st = check_splits(num_q_heads, lay->num_kv_heads, max_splits);
  if (st != OSCAR_OK) return st;
  if (!valid_scale(sm_scale)) return OSCAR_ERR_INVALID_ARGUMENT;
  if (batch == 0) return OSCAR_OK;
  if (!pages || !block_table || !q || !seq_lens || !workspace) return OSCAR_ERR_INVALID_ARGUMENT;
  if (!aligned16(pages) || !aligned16(q) || !aligned16(workspace)) return OSCAR_ERR_INVALID_ARGUMENT;
  if (workspace_bytes_given < workspace_bytes(batch, num_q_heads, max_splits))
    return OSCAR_ERR_WORKSPACE_TOO_SMALL;
  Workspace ws = make_workspace(workspace, batch, num_q_heads, max_splits);
  return hip_status(launch_bf16_decode(geom(lay), pages, block_table, batch, num_q_heads, q,
                                       seq_lens, sm_scale, split_pages, ws, (hipStream_t)stream));
}

int32_t oscar_mfma_bf16_tiles(const uint16_t* a, const uint16_t* b, const float* c, float* d,
                              int32_t tiles, void* stream) {
  if (tiles < 0 || tiles > (1 << 20)) return OSCAR_ERR_INVALID_ARGUMENT;
  if (tiles == 0) return OSCAR_OK;
  if (!a || !b || !c || !d) return OSCAR_ERR_INVALID_ARGUMENT;
  return hip_status(launch_mfma_bf16_tiles(a, b, c, d, tiles, (hipStream_t)stream));
}

int32_t oscar_read_records(const uint8_t* pool, int32_t num_records, const int32_t* record_ids,
                           int32_t n, int32_t num_workers, uint32_t* out, void* stream) {
  if (n < 0 || num_records < 1 || num_workers < 1 || num_workers > kMaxWorkers)
    return OSCAR_ERR_INVALID_ARGUMENT;
  if (n == 0) return OSCAR_OK;
  if (!pool || !record_ids || !out || !aligned16(pool)) return OSCAR_ERR_INVALID_ARGUMENT;
  return hip_status(launch_read_records(pool, num_records, record_ids, n, num_workers, out,
                                        (hipStream_t)stream));
}

}  // extern "C"
