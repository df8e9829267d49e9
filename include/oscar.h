/*
 * oscar.h - C ABI of the rotated INT2 KV cache and its mixed-precision paged decode attention
 * for AMD Instinct MI355X (gfx950).
 *
 * The method: every cached key/value row is multiplied by a fixed, offline-derived orthogonal
 * rotation, clipped with fixed thresholds and stored in 2 bits per element inside a paged KV
 * cache, while a few initial "sink" tokens and a recent window of tokens stay in BF16; decode
 * attention reads the three parts in one fused softmax.  Sources: OSCAR project card
 * "FutureMLS-Lab/OSCAR" (agentlenshq.com), section "How it works"; OSCAR paper
 * (thelatestinai.com/papers/2605.17757), "Abstract"; write-up "OSCAR: Cut LLM Inference Costs
 * 8x with 2-bit KV Cache Quantization" (strixaai.com), sections "Practical Summary" and
 * "How OSCAR Works".
 *
 * Conventions for every entry point
 *   - Array arguments are DEVICE pointers (memory on the GPU that is current when the call is
 *     made), except `lay`, which is a host pointer read during the call only.
 *   - The caller owns all memory.  The library never allocates, frees or keeps a pointer past
 *     the call.  Its only state between calls is a per-device cache of the compute-unit count
 *     and of the device address of oscar_decode_attention_static's workspace.
 *   - Every call enqueues its kernels on `stream` (a hipStream_t; NULL = the default stream)
 *     and returns without synchronising.  Calls on one stream run in order; calls that write
 *     the same cache from two streams at once race.
 *   - Host-visible arguments are checked before anything is launched; on a non-zero return
 *     nothing was launched.  OSCAR_ERR_HIP reports a launch failure (hipGetLastError).
 *   - Values that live in device memory (lengths, positions, block-table entries, slot ids)
 *     are not checked by the host.  The kernels skip any page id outside [0, num_pages), any
 *     logical page outside the block-table row and any slot outside [0, num_slots) instead of
 *     touching memory outside the caller's buffers; results for such inputs are unspecified.
 *   - Inputs must be finite, and every rotated value must stay below 65504 in magnitude so the
 *     fp16 scales and zeros stay finite.
 *   - Pointers to pages, stores, q, k_new, v_new and workspace must be 16-byte aligned.
 *   - Size limits (else OSCAR_ERR_UNSUPPORTED): batch * num_q_heads at most 2^27 for the decode,
 *     combine and workspace calls; total_new at most 2^30 for the appends.  Every size the
 *     library derives from them then fits its int32 grids and indices.
 *
 * Fixed geometry: head_dim 128, page_size 16 tokens, quantisation group 32 channels.
 *
 * INT2 page record (one per physical page and KV head, 1536 bytes, all fields little-endian):
 *   [   0,  512) K codes.  Channel c of page slot r (token r of the page) belongs to 16-channel
 *                word d = c/16, stored as the dword at 8*(16*(d%4) + r) + 4*(d/4); inside the
 *                dword, byte (c%16)/4, bits 2*(c%4)..+1.
 *   [ 512, 1024) V codes.  Channel c of slot r: chunk L = 16*(r/4) + c%16 at 512 + 8*L;
 *                dword (r%4)/2 of the chunk, 16-bit half r%2; bits 2*(c/16)..+1 of the half.
 *   [1024, 1280) K scale/zero: group g of slot r at 1024 + 16*r + 4*g, fp16 scale then fp16 zero.
 *   [1280, 1536) V scale/zero, same arrangement at 1280 + 16*r + 4*g.
 *   A code q in group g decodes to scale_g * q + zero_g, in the rotated frame.
 *   Pool: uint8 [num_pages][num_kv_heads][1536].
 *
 * BF16 sink/window store: uint16 (bf16 bits) [num_slots][num_kv_heads][S+W][2][128], rotated
 *   K (index 0) and V (index 1).  Sink position p < S lives in row p; a window position p >= S
 *   lives in row S + (p mod W).
 *
 * Block table: int32 [batch][max_pages_per_seq]; entry [b][i] is the physical page holding
 *   positions 16*i .. 16*i+15 of sequence b.  Unused entries should be -1.
 */
#ifndef OSCAR_H_
#define OSCAR_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  OSCAR_OK = 0,
  OSCAR_ERR_INVALID_ARGUMENT = 1,   /* null pointer, negative size, bad ratio, ... */
  OSCAR_ERR_UNSUPPORTED = 2,        /* geometry other than 128 / 16 / 32, too many heads */
  OSCAR_ERR_WORKSPACE_TOO_SMALL = 3,
  OSCAR_ERR_HIP = 4                 /* a kernel launch failed */
};

typedef struct oscar_layout {
  int32_t num_kv_heads;       /* Hkv >= 1 */
  int32_t head_dim;           /* must be 128 */
  int32_t page_size;          /* must be 16 */
  int32_t group_size;         /* must be 32 */
  int32_t num_sink;           /* S >= 0 */
  int32_t window;             /* W >= 0; S + W <= 256 */
  int32_t num_pages;          /* physical pages in the pool */
  int32_t max_pages_per_seq;  /* block-table row stride */
  int32_t num_slots;          /* sequences the BF16 sink/window store can hold */
} oscar_layout;

/* Human-readable name of a status code (static storage). */
const char* oscar_status_string(int32_t status);

/*
 * Rotate, clip, quantise and append new K/V rows to the cache.
 * (OSCAR project card, "How it works": fixed per-layer rotations and clipping thresholds, INT2
 *  bulk with BF16 sinks and recent window; OSCAR paper, "Abstract": INT2 kernel compatible
 *  with a paged KV cache.)
 *
 * For sequence b, rows new_offsets[b] .. new_offsets[b+1]-1 of k_new / v_new are its new
 * tokens, at positions start_pos[b], start_pos[b]+1, ...  For every new row x of KV head h:
 *   y = x . R (R = rot_k[h] or rot_v[h]; row-vector convention), computed as an fp64 sum over
 *       the 128 input channels in ascending order, rounded once to fp32;
 *   for each 32-channel group of y: mx, mn = max, min; mx_c = clip*mx, mn_c = clip*mn (fp32);
 *       scale = fp16(fp32(mx_c - mn_c) / 3), zero = fp16(mn_c) (round to nearest even);
 *   code = clamp(rint((y - zero) / scale), 0, 3) in fp32 (0 when scale == 0).
 * Every new position's codes and scales go to its page record; a position p with p < S, or
 * p >= start_pos[b] + n_new - W, also gets bf16(y) in the sink/window store row of slot
 * slot_ids[b] (slot b when slot_ids is NULL).
 *
 *   lay          host; geometry and pool sizes.
 *   pages        uint8 [num_pages][Hkv][1536], written.
 *   sinkwin      uint16 [num_slots][Hkv][S+W][2][128], written (may be NULL when S + W == 0).
 *   block_table  int32 [batch][max_pages_per_seq].
 *   slot_ids     int32 [batch] or NULL.
 *   batch        number of sequences (>= 0; 0 launches nothing).
 *   total_new    rows in k_new / v_new (== new_offsets[batch]; >= 0).
 *   k_new, v_new bf16 bits [total_new][Hkv][128], unrotated (after RoPE).
 *   new_offsets  int32 [batch+1], non-decreasing, new_offsets[0] == 0.
 *   start_pos    int32 [batch].
 *   rot_k, rot_v fp32 [Hkv][128][128], row-major.
 *   clip_k, clip_v  clip ratios, 0 < clip <= 1.
 * Two new rows of one call must not share a (page, slot).
 */
int32_t oscar_rotate_quantize_append(
    const oscar_layout* lay, uint8_t* pages, uint16_t* sinkwin,
    const int32_t* block_table, const int32_t* slot_ids,
    int32_t batch, int32_t total_new,
    const uint16_t* k_new, const uint16_t* v_new,
    const int32_t* new_offsets, const int32_t* start_pos,
    const float* rot_k, const float* rot_v, float clip_k, float clip_v,
    void* stream);

/* Kernel choices for oscar_rotate_quantize_append_ex. */
enum {
  OSCAR_APPEND_AUTO = 0,    /* the matrix cores from 256 new rows, else the vector ALUs */
  OSCAR_APPEND_VECTOR = 1,  /* the rotation in fp64 on the vector ALUs, as defined above */
  OSCAR_APPEND_MATRIX = 2   /* the rotation on the bf16 matrix cores (R split exactly into three
                               bf16 pieces), each rotated value's error bounded; every scale,
                               zero, code and BF16 copy the bound cannot certify is recomputed
                               as defined above */
};

/*
 * oscar_rotate_quantize_append with two more arguments.
 *
 * k_mean (NULLABLE, fp32 [Hkv][128], 4-byte aligned): a fixed per-(KV head, channel) key mean
 * removed before the key rotation, the attention-equivalent key reparameterisation of the
 * OptR abstract on the OSCAR paper's page ("OSCAR: Offline Spectral Covariance-Aware Rotation
 * for 2-bit KV Cache Quantization"): q . (k - mu) differs from q . k by q . mu for every
 * position, so attention outputs are unchanged while the keys lose their channel offsets.
 * For K rows the rotated value becomes
 *   y_j = fp32( S_j - C_j ),  S_j = the fp64 ascending sum above,
 *                             C_j = sum_i mu_i R_ij in fp64, i ascending from +0.0,
 * with the subtraction in fp64; V rows are unchanged.  NULL is the plain rotation, byte for
 * byte.  The same mean must be used for every append of a cache.  The decode entry points do
 * not take it: their outputs are unchanged, and the log-sum-exp oscar_combine reports is the
 * one of the centered logits (lower by sm_scale * (q . mu) for each query head).
 *
 * method: one of OSCAR_APPEND_* (anything else is OSCAR_ERR_INVALID_ARGUMENT).  Every method
 * writes the same bytes; they differ in speed only (the matrix cores win for prefill-sized
 * appends, the vector ALUs for a few rows).  oscar_rotate_quantize_append is this call with
 * k_mean NULL and OSCAR_APPEND_AUTO.
 */
int32_t oscar_rotate_quantize_append_ex(
    const oscar_layout* lay, uint8_t* pages, uint16_t* sinkwin,
    const int32_t* block_table, const int32_t* slot_ids,
    int32_t batch, int32_t total_new,
    const uint16_t* k_new, const uint16_t* v_new,
    const int32_t* new_offsets, const int32_t* start_pos,
    const float* rot_k, const float* rot_v, const float* k_mean, float clip_k, float clip_v,
    int32_t method, void* stream);

/*
 * oscar_rotate_quantize_append with the Hadamard rotation R = diag(s) . H / sqrt(128) (H the
 * Sylvester-Hadamard matrix of order 128, H_ij = (-1)^popcount(i & j), s a fixed sign per input
 * channel) for both K and V: the rotation the OSCAR paper's page ("OSCAR: Offline Spectral
 * Covariance-Aware Rotation for 2-bit KV Cache Quantization", OSCAR and INT4 abstracts) names as
 * the simple outlier-reducing baseline.  For every new row x:
 *   u_i = -x_i where signs[h][i] < 0, else x_i;
 *   T = fast Walsh-Hadamard transform of u in fp64, stages h = 1, 2, 4, ..., 64, the pair
 *       (u_i, u_{i+h}) (i in the lower half of its block) becoming (u_i + u_{i+h}, u_i - u_{i+h});
 *   y_j = fp32( fp64(T_j * r) ), r = the double nearest to 1/sqrt(128);
 * then the same groups, scales, zeros, codes, records and BF16 copies as
 * oscar_rotate_quantize_append.  No matrix is read.  Attention over such a cache takes the dense
 * fp32 form R_ij = fp32(s_i H_ij r) as rot_k (oscar_decode_attention) and rot_v (oscar_combine).
 *
 *   signs_k, signs_v  NULLABLE int8 [Hkv][128] (device); NULL means every sign +1.
 * Other arguments, validation and errors as oscar_rotate_quantize_append.
 */
int32_t oscar_rotate_quantize_append_hadamard(
    const oscar_layout* lay, uint8_t* pages, uint16_t* sinkwin,
    const int32_t* block_table, const int32_t* slot_ids,
    int32_t batch, int32_t total_new,
    const uint16_t* k_new, const uint16_t* v_new,
    const int32_t* new_offsets, const int32_t* start_pos,
    const int8_t* signs_k, const int8_t* signs_v, float clip_k, float clip_v,
    void* stream);

/*
 * INT4 variant of the cache: the same rotation (with the optional key mean of
 * oscar_rotate_quantize_append_ex), clip, 32-channel groups, fp16 scale/zero and BF16
 * sink/window store, with 16-level codes: s = fp16(fp32(c*mx - c*mn) / 15), z = fp16(c*mn),
 * code = clamp(rint((y - z) / s), 0, 15) (0 when s == 0).  Token-wise INT4 with a rotation is the
 * serving-compatible 4-bit design of the INT4 abstract on the OSCAR paper's page ("OSCAR:
 * Offline Spectral Covariance-Aware Rotation for 2-bit KV Cache Quantization").
 * The pool is uint8 [num_pages][Hkv][2560]; within a record (slot r, channel c, group g; 4-bit
 * codes, an arrangement made for matrix-core operands):
 *   [   0, 1024)  K codes in 16-byte chunks: chunk 16*q + r holds slot r's channels 16q..16q+15
 *                 and 64+16q..64+16q+15; with h = c/64, q = (c%64)/16, j = c%16, i = j%4,
 *                 channel c is at byte 16*(16q + r) + 8h + 4*(i/2) + j/4, bits 4*(i%2);
 *   [1024, 2048)  V codes in 16-byte chunks: chunk 16*(r/4) + c%16; with nb = c/16, u = r%4,
 *                 channel c is at byte 1024 + 16*chunk + 4*(nb/2) + 2*(u%2) + u/2, bits
 *                 4*(nb%2) (each slot owns whole bytes);
 *   [2048, 2304)  K (fp16 scale, fp16 zero) at 2048 + 16*r + 4*g;
 *   [2304, 2560)  V (scale, zero) at 2304 + 16*r + 4*g.
 * Arguments, validation and errors as oscar_rotate_quantize_append_ex, with no method argument:
 * the choice is always that of OSCAR_APPEND_AUTO (the fp64 vector-ALU rotation below 256 new
 * rows, from 256 the certified matrix-core one, which recomputes in fp64 every value whose code
 * its bound cannot decide); both write the same bytes.
 */
int32_t oscar_int4_rotate_quantize_append(
    const oscar_layout* lay, uint8_t* pages, uint16_t* sinkwin,
    const int32_t* block_table, const int32_t* slot_ids,
    int32_t batch, int32_t total_new,
    const uint16_t* k_new, const uint16_t* v_new,
    const int32_t* new_offsets, const int32_t* start_pos,
    const float* rot_k, const float* rot_v, const float* k_mean, float clip_k, float clip_v,
    void* stream);

/*
 * Decode attention over an INT4 cache, written in the workspace format of
 * oscar_decode_attention and finished by oscar_combine with the same rot_v.  The work split of
 * oscar_decode_attention (equal runs of INT4 pages per worker wavefront, one per resident slot;
 * at most max_splits partials per (sequence, KV head); the BF16 sink/window positions as extra
 * partials), on the matrix cores for every G = num_q_heads / Hkv (1, 2, 4 or 8).
 * Arguments, validation and errors as oscar_decode_attention, with split_pages (>= 1, kept for
 * compatibility and not used) in place of num_workers.
 */
int32_t oscar_int4_decode_attention(
    const oscar_layout* lay, const uint8_t* pages, const uint16_t* sinkwin,
    const int32_t* block_table, const int32_t* slot_ids,
    int32_t batch, int32_t num_q_heads,
    const uint16_t* q, const int32_t* seq_lens, const float* rot_k, float sm_scale,
    int32_t split_pages, int32_t max_splits,
    void* workspace, size_t workspace_bytes, void* stream);

/*
 * Bytes of workspace oscar_decode_attention / oscar_bf16_decode_attention need for `batch`
 * sequences of `num_q_heads` query heads split at most `max_splits` ways: per (sequence, query
 * head) a 1024-byte query block and max_splits + 8 partial slots of 520 bytes (128 fp32
 * outputs, then (m, l) in a region of its own), plus a plan of 4 * (4 + 3 * batch +
 * batch * num_q_heads) bytes rounded up to 256.  Returns 0 for invalid arguments, for
 * max_splits above 65535 and for batch * num_q_heads above 2^27.
 */
size_t oscar_decode_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t max_splits);

/*
 * Mixed-precision paged decode attention, first stage: per (sequence, KV head, split) partial
 * softmax results, written to `workspace`.  oscar_combine finishes the step.
 * (OSCAR project card, "How it works": BF16 sink + recent window + INT2 bulk under fused
 *  mixed-precision flash attention; OSCAR paper, "Abstract": paged INT2 attention kernel.)
 *
 * For sequence b of length L = seq_lens[b] (positions 0..L-1, including the token being
 * decoded) and query head j of KV head h = j / (num_q_heads / Hkv):
 *   q' = q[b][j] . rot_k[h];
 *   positions [0, min(L,S)) and the last min(W, L - min(L,S)) positions are read from the
 *   BF16 store; the others are decoded from their INT2 records;
 *   logits z_p = sm_scale * (q' . k_p), and the partials hold, per split, the max of
 *   z_p*log2(e), the sum of 2^(z_p*log2(e) - max), and the matching unnormalised weighted sum
 *   of the rotated values.
 * Work split: the INT2 pages of all (sequence, KV head) pairs, laid end to end in (sequence,
 * head) order, are cut into equal runs of C pages, one per worker wavefront, so every worker
 * streams the same number of pages however the lengths are mixed.  A run yields one partial
 * for each pair it touches; a pair's partials fill its slots 0, 1, ... in page order.  C is the
 * smallest run length that needs at most num_workers runs and gives no pair more than
 * max_splits partials.  The BF16 positions of each pair (sink first, then window, in position
 * order) form up to 8 more partials, the pair's window slots: one for all of them when the
 * launch has at least half as many (sequence, KV head) pairs as the device has compute units,
 * else one per 32 positions (each on its own workgroup, so that a short launch is not held up
 * by the window's dependent loads); unused window slots are marked empty.
 *
 *   q            bf16 bits [batch][num_q_heads][128] (after RoPE, unrotated).
 *   seq_lens     int32 [batch], >= 1.
 *   rot_k        fp32 [Hkv][128][128].
 *   sm_scale     softmax scale, usually 1/sqrt(128); finite and > 0 (else
 *                OSCAR_ERR_INVALID_ARGUMENT).
 *   num_workers  worker wavefronts, 0 for one per resident wavefront slot of the device
 *                (the fastest choice); at most 2^20.
 *   max_splits   INT2 partials per (sequence, KV head), >= 1, with
 *                8 * (num_q_heads / Hkv) * (max_splits + 8) <= 49152 (else
 *                OSCAR_ERR_UNSUPPORTED).  Too small a value lengthens the runs.
 *   workspace    device buffer of at least oscar_decode_workspace_bytes(batch, num_q_heads,
 *                max_splits) bytes; contents on entry do not matter.
 * batch * Hkv * max_pages_per_seq must be below 2^31 (else OSCAR_ERR_UNSUPPORTED).
 * A block-table entry outside [0, num_pages) for a position below seq_lens[b] is a caller error:
 * the pool's last page is read in its place (memory stays in bounds; the result is
 * unspecified).
 * num_q_heads must be a multiple of Hkv with num_q_heads / Hkv in {1, 2, 4, 8}.
 */
int32_t oscar_decode_attention(
    const oscar_layout* lay, const uint8_t* pages, const uint16_t* sinkwin,
    const int32_t* block_table, const int32_t* slot_ids,
    int32_t batch, int32_t num_q_heads,
    const uint16_t* q, const int32_t* seq_lens, const float* rot_k, float sm_scale,
    int32_t num_workers, int32_t max_splits,
    void* workspace, size_t workspace_bytes, void* stream);

/*
 * The two halves of oscar_decode_attention, for callers that overlap the query preparation
 * with other work, such as the new token's append on a second stream (the two are independent;
 * the decode needs both).  oscar_prepare_queries computes q' = q . rot_k with its int8 encoding
 * and the work plan into `workspace`; oscar_decode_attention_prepared then runs the attention
 * over the cache from them.  The pair, called in this order, computes exactly what
 * oscar_decode_attention computes (the same kernels: results are identical).  The second call
 * must get the same layout, batch, num_q_heads, seq_lens contents, num_workers, max_splits and
 * workspace as the first and be ordered after it, and after every append it should see; the
 * workspace must not be reused in between.  Arguments, validation and errors as
 * oscar_decode_attention (each call checks the arguments it takes).
 * (OSCAR project card, "How it works": rotated queries against the rotated cache; OSCAR paper,
 *  "Abstract": paged INT2 attention kernel.)
 */
int32_t oscar_prepare_queries(
    const oscar_layout* lay, int32_t batch, int32_t num_q_heads,
    const uint16_t* q, const int32_t* seq_lens, const float* rot_k,
    int32_t num_workers, int32_t max_splits,
    void* workspace, size_t workspace_bytes, void* stream);

int32_t oscar_decode_attention_prepared(
    const oscar_layout* lay, const uint8_t* pages, const uint16_t* sinkwin,
    const int32_t* block_table, const int32_t* slot_ids,
    int32_t batch, int32_t num_q_heads, const int32_t* seq_lens, float sm_scale,
    int32_t num_workers, int32_t max_splits,
    void* workspace, size_t workspace_bytes, void* stream);

/*
 * The front half of a decode step in one launch: this step's new K/V rows appended as
 * oscar_rotate_quantize_append_ex does with OSCAR_APPEND_AUTO (the arguments lay ... clip_v,
 * k_mean optional), and the queries prepared as oscar_prepare_queries does (num_q_heads, q,
 * seq_lens, rot_k, num_workers, max_splits, workspace).  One `batch` serves both: the step's
 * sequences, whose new_offsets / start_pos place the new rows and whose seq_lens are the lengths
 * after the append.  The two parts are independent and each alone leaves most of the device
 * idle, so with fewer than 256 new rows (the append's 4-row vector kernel) their workgroups
 * run in one launch; from 256 rows on they are two launches.  Either way the call writes
 * exactly the bytes of oscar_rotate_quantize_append_ex followed by oscar_prepare_queries, and
 * oscar_decode_attention_prepared continues it.  total_new = 0 prepares the queries only.
 * Validation and errors: the union of those two calls' (the append's pointers only when
 * total_new > 0).  (OSCAR project card, "How it works": K/V rows rotated, clipped and stored in
 * INT2 beside the BF16 sink and window, queries rotated by the same R_K.)
 */
int32_t oscar_append_and_prepare(
    const oscar_layout* lay, uint8_t* pages, uint16_t* sinkwin,
    const int32_t* block_table, const int32_t* slot_ids,
    int32_t batch, int32_t total_new,
    const uint16_t* k_new, const uint16_t* v_new,
    const int32_t* new_offsets, const int32_t* start_pos,
    const float* rot_k, const float* rot_v, const float* k_mean, float clip_k, float clip_v,
    int32_t num_q_heads, const uint16_t* q, const int32_t* seq_lens,
    int32_t num_workers, int32_t max_splits,
    void* workspace, size_t workspace_bytes, void* stream);

/*
 * Second stage: merge the splits of every (sequence, query head) in ascending split order,
 * normalise, and rotate back with the transpose of the value rotation:
 *   M = max_s m_s, l = sum_s 2^(m_s - M) l_s, o' = sum_s 2^(m_s - M) o'_s / l,
 *   out = o' . rot_v[h]^T,  lse = M*ln(2) + ln(l)  (natural-log sum of exp of the logits).
 * (OSCAR paper, "Abstract": attention stays exact under the fixed orthogonal rotation.)
 *
 *   workspace  as written by oscar_decode_attention / oscar_bf16_decode_attention with the
 *              same batch, num_q_heads and max_splits.
 *   rot_v      fp32 [Hkv][128][128], or NULL for no rotation (BF16 baseline).
 *   out        fp32 [batch][num_q_heads][128], written.
 *   lse        fp32 [batch][num_q_heads] or NULL.
 * A row with no positions gets out = 0 and lse = -inf.
 */
int32_t oscar_combine(
    int32_t batch, int32_t num_q_heads, int32_t num_kv_heads, int32_t max_splits,
    const void* workspace, size_t workspace_bytes, const float* rot_v,
    float* out, float* lse, void* stream);

/*
 * BF16 paged baseline in the same library: no rotation, no quantisation.  The pages' memory,
 * throughput and latency claims are all stated against a BF16 KV cache (write-up, "Practical
 * Summary"; OSCAR paper, "Abstract").
 *
 * BF16 page (one per physical page and KV head, 8192 bytes): K as bf16 [16 tokens][128],
 * then V transposed as bf16 [128 channels][16 tokens].  Pool: uint16 [num_pages][Hkv][4096].
 * Only num_kv_heads, head_dim, page_size, num_pages and max_pages_per_seq of `lay` are used.
 */
int32_t oscar_bf16_append(
    const oscar_layout* lay, uint16_t* pages, const int32_t* block_table,
    int32_t batch, int32_t total_new, const uint16_t* k_new, const uint16_t* v_new,
    const int32_t* new_offsets, const int32_t* start_pos, void* stream);

/*
 * BF16 baseline decode, first stage: the same workspace format as oscar_decode_attention
 * over all positions [0, L) of the BF16 pages (q unrotated), split per sequence into runs of
 * split_pages logical pages (split s covers pages [s*split_pages, (s+1)*split_pages), the last
 * split everything after); finish with oscar_combine(..., rot_v = NULL, ...).
 */
int32_t oscar_bf16_decode_attention(
    const oscar_layout* lay, const uint16_t* pages, const int32_t* block_table,
    int32_t batch, int32_t num_q_heads, const uint16_t* q, const int32_t* seq_lens,
    float sm_scale, int32_t split_pages, int32_t max_splits,
    void* workspace, size_t workspace_bytes, void* stream);

/*
 * Decode attention and combine in one call with no allocation anywhere: for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  It computes exactly what oscar_decode_attention followed by oscar_combine
 * compute (same kernels, same work plan for the same num_workers and max_splits, so the same
 * bits), with the decode workspace in a buffer that the library holds in device memory on each
 * GPU it runs on, OSCAR_STATIC_WORKSPACE_BYTES in size, for the life of the process.
 *   Arguments as for oscar_decode_attention and oscar_combine (rot_v, out, lse); there is no
 *   workspace argument.
 * Returns OSCAR_ERR_WORKSPACE_TOO_SMALL when oscar_decode_workspace_bytes(batch, num_q_heads,
 * max_splits) exceeds OSCAR_STATIC_WORKSPACE_BYTES (a smaller max_splits lengthens the worker
 * runs and needs less), and OSCAR_ERR_HIP if the buffer's device address cannot be looked up;
 * nothing is launched in either case.  The buffer's address is looked up once per device, on
 * the first call with that device current.  The buffer keeps the last call's contents, and the
 * kernels read nothing in it that the same call has not written.  All calls on one GPU share
 * its buffer: calls whose executions overlap on one GPU (on different streams, or from
 * different threads without ordering) race and give undefined results.
 */
#define OSCAR_STATIC_WORKSPACE_BYTES ((size_t)32 << 20)
int32_t oscar_decode_attention_static(
    const oscar_layout* lay, const uint8_t* pages, const uint16_t* sinkwin,
    const int32_t* block_table, const int32_t* slot_ids,
    int32_t batch, int32_t num_q_heads,
    const uint16_t* q, const int32_t* seq_lens, const float* rot_k, const float* rot_v,
    float sm_scale, int32_t num_workers, int32_t max_splits,
    float* out, float* lse, void* stream);

/*
 * Accumulation check of the matrix-core instruction (not part of the method): for each of
 * `tiles` independent tiles, one v_mfma_f32_16x16x32_bf16 computes D = A . B + C.  The
 * matrix-core prefill append (oscar_rotate_quantize_append from 256 rows on) certifies its
 * bytes with an error bound of that instruction's fp32 accumulation (per instruction at most
 * 11u * sum_k |A[m][k] B[k][n]| + 4u |C[m][n]| + 2^-124, u = 2^-24: four 8-product passes,
 * each dropping the bits below 2^-24 of its largest product and rounding the accumulator to
 * nearest once); this entry point lets a test re-measure that on the device at hand.
 *   a  bf16 bits [tiles][16][32] row-major;  b  bf16 bits [tiles][32][16] row-major;
 *   c  fp32 [tiles][16][16];  d  fp32 [tiles][16][16], written.
 * Returns OSCAR_ERR_INVALID_ARGUMENT for tiles outside [0, 2^20] or a null pointer.
 */
int32_t oscar_mfma_bf16_tiles(const uint16_t* a, const uint16_t* b, const float* c, float* d,
                              int32_t tiles, void* stream);

/*
 * Read-bandwidth probe (a measurement aid, not part of the method): reads the INT2 records
 * pool + 1536 * record_ids[i], i = 0..n-1, with the decode kernel's access pattern and none of
 * its arithmetic, so that the HBM rate it reaches is the practical ceiling of the decode
 * kernel's INT2 stream on the device.  A record index is page * num_kv_heads + head.
 * Wavefront w of num_workers reads the w-th of num_workers equal runs of the list, two
 * records per step, and writes the XOR of all 32-bit words it read, folded per lane, to
 * out[64*w + lane].
 *   pool        uint8 INT2 pool of num_records records (16-byte aligned)
 *   num_records records in the pool (num_pages * num_kv_heads); a record id outside
 *               [0, num_records) reads the last record instead, so memory stays in bounds
 *   record_ids  int32 [n]
 *   out         uint32 [64 * num_workers], written
 * A run of odd length folds its last record once (the step's second record contributes zero).
 * Returns OSCAR_ERR_INVALID_ARGUMENT for n < 0, num_records < 1, num_workers outside
 * [1, 1048576] or a null/misaligned pointer.
 */
int32_t oscar_read_records(const uint8_t* pool, int32_t num_records, const int32_t* record_ids,
                           int32_t n, int32_t num_workers, uint32_t* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* OSCAR_H_ */
