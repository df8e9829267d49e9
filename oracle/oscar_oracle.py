"""CPU oracle for the rotated-INT2 KV cache and its mixed-precision decode attention.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's CPU-baseline
leg may import this module.  The HIP library never calls it and it never calls the library;
the two share no code.  Everything here is plain numpy, written to be checked by eye against
the method's description, not to be fast.

What it follows.  The OSCAR pages (project card "FutureMLS-Lab/OSCAR", section "How it works";
the write-up "OSCAR: Cut LLM Inference Costs 8x with 2-bit KV Cache Quantization", sections
"Practical Summary" and "How OSCAR Works"; and the OSCAR paper's "Abstract") fix the shape of
the method:

  * every cached K/V row is multiplied by a fixed orthogonal rotation, clipped with fixed
    thresholds, and quantised to 2 bits (4 levels);
  * a few initial "sink" tokens and a recent window of tokens are kept in BF16, the rest of
    the cache in INT2, inside a paged KV cache;
  * decode attention reads that mixed cache in one fused softmax.

Every number and bit-level choice the pages leave open is taken from the workload
definitions and the readings listed in the design notes: per-token groups of 32 channels,
asymmetric (min/scale) levels with fp16 scale and zero, clip ratio applied to each group's
min and max, 16-token pages, q rotated by the key rotation and the output rotated back by
the transpose of the value rotation.

Precision.  Rotations and attention are fp64.  The quantiser parameters are an fp32 formula
(numpy float32 scalars and arrays: IEEE single, round to nearest even, never fused), then
rounded to fp16 with round to nearest even, because the encoded bytes must be reproduced bit
for bit.  bf16 rounding is round to nearest even.

Parity pins: every function here is checked in the CPU tests against closed forms,
invariants, special cases and brute force (orthogonality, rotation invariance of attention,
level membership, exhaustive code enumeration, hand-derived record bytes, partition
invariance of the split merge; for the key-mean form, one rounded subtraction under identity
and signed-permutation rotations, exact rational sums, and softmax invariance).  No function
is "parity unpinned".
"""
from __future__ import annotations

import numpy as np

D = 128          # head dimension
PAGE = 16        # tokens per page
GROUP = 32       # channels per quantisation group
NGROUPS = D // GROUP
LEVELS = 4       # 2-bit codes
RECORD = 1536    # bytes of one (page, KV head) INT2 record
K_CODES, V_CODES, K_META, V_META = 0, 512, 1024, 1280


# ----------------------------------------------------------------------------------------
# Rounding helpers (own implementations; the input generator has its own copies).
# ----------------------------------------------------------------------------------------

def f32_to_bf16_bits(x) -> np.ndarray:
    """Round float32 to bf16 with round-to-nearest-even; returns uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    return ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)


def bf16_bits_to_f64(b) -> np.ndarray:
    u = np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


# ----------------------------------------------------------------------------------------
# Rotation of cache rows and of the query.
# ----------------------------------------------------------------------------------------

def rotate_rows(x_bits: np.ndarray, rot32: np.ndarray) -> np.ndarray:
    """y = x . R for bf16 rows x (row-vector convention), result rounded to fp32.

    The sum over the 128 input channels is accumulated in fp64 in ascending channel order
    starting from +0.0, then rounded once to fp32 (nearest even).  Each product of a bf16
    value and an fp32 value is exact in fp64, so the order of the additions is the only
    rounding choice, and it is fixed here.

    x_bits: uint16 [N][128] bf16 bit patterns.  rot32: float32 [128][128].
    Returns float32 [N][128].
    """
    x = bf16_bits_to_f64(x_bits)
    r = np.asarray(rot32, dtype=np.float32).astype(np.float64)
    acc = np.zeros((x.shape[0], D), dtype=np.float64)
    for i in range(D):
        acc = acc + x[:, i:i + 1] * r[i:i + 1, :]
    return acc.astype(np.float32)


def mean_shift(mean32: np.ndarray, rot32: np.ndarray) -> np.ndarray:
    """C = mu . R for a per-channel key mean mu (fp32 [128]): fp64, ascending input channel,
    from +0.0 (each product of two fp32 values is exact in fp64).  Returns fp64 [128]."""
    mu = np.asarray(mean32, dtype=np.float32).astype(np.float64)
    r = np.asarray(rot32, dtype=np.float32).astype(np.float64)
    acc = np.zeros(D, dtype=np.float64)
    for i in range(D):
        acc = acc + mu[i] * r[i]
    return acc


def rotate_rows_centered(x_bits: np.ndarray, rot32: np.ndarray, mean32) -> np.ndarray:
    """y = (x - mu) . R for bf16 key rows, with a fixed per-channel mean mu subtracted.

    The OptR abstract on the OSCAR paper's page ("OSCAR: Offline Spectral Covariance-Aware
    Rotation for 2-bit KV Cache Quantization") adds an attention-equivalent reparameterisation
    of the keys that removes large per-channel offsets: q . (k - mu) differs from q . k by
    q . mu, the same for every position of a query, so the softmax does not change.  Reading
    taken here: mu is a fixed fp32 vector per KV head, removed in the rotated frame as
        y_j = fp32( fp64(S_j - C_j) ),  S_j = the sum of rotate_rows, C_j = mean_shift(mu, R)_j,
    one fp64 subtraction then one rounding to fp32.  mean32 None gives rotate_rows exactly.
    """
    if mean32 is None:
        return rotate_rows(x_bits, rot32)
    x = bf16_bits_to_f64(x_bits)
    r = np.asarray(rot32, dtype=np.float32).astype(np.float64)
    acc = np.zeros((x.shape[0], D), dtype=np.float64)
    for i in range(D):
        acc = acc + x[:, i:i + 1] * r[i:i + 1, :]
    return (acc - mean_shift(mean32, rot32)[None, :]).astype(np.float32)


# Hadamard rotation: R = diag(s) . H / sqrt(128), H the Sylvester-Hadamard matrix of order 128
# (H_ij = (-1)^popcount(i & j)) and s a fixed sign per input channel.  The paper's page ("OSCAR:
# Offline Spectral Covariance-Aware Rotation for 2-bit KV Cache Quantization", the OSCAR and
# INT4 abstracts) names Hadamard transforms as the simple rotation that reduces outliers
# (block-diagonal in the INT4 work).  Reading taken here for its arithmetic: the signed row goes
# through the fast Walsh-Hadamard transform in fp64 (stages h = 1, 2, 4, ..., 64; the pair
# (a, b) = (u_i, u_{i+h}) becomes (a + b, a - b)), each result is multiplied in fp64 by the
# double nearest to 1/sqrt(128), and rounded once more to fp32.

HADAMARD_SCALE = float(np.sqrt(np.float64(2.0)) / 16.0)   # nearest double to 2^-3.5


def fwht(u: np.ndarray) -> np.ndarray:
    """Unnormalised fast Walsh-Hadamard transform of fp64 rows [N][128], stage by stage."""
    v = np.array(u, dtype=np.float64, copy=True)
    h = 1
    while h < D:
        for start in range(0, D, 2 * h):
            a = v[:, start:start + h].copy()
            b = v[:, start + h:start + 2 * h].copy()
            v[:, start:start + h] = a + b
            v[:, start + h:start + 2 * h] = a - b
        h *= 2
    return v


def rotate_rows_hadamard(x_bits: np.ndarray, signs) -> np.ndarray:
    """y = x . diag(s) H / sqrt(128) for bf16 rows: fp64 FWHT of the signed row, times
    HADAMARD_SCALE in fp64, rounded to fp32.  signs: [128] of +-1 (a negative entry flips the
    channel) or None for all +1.  Returns float32 [N][128]."""
    x = bf16_bits_to_f64(x_bits)
    if signs is not None:
        x = x * np.where(np.asarray(signs) < 0, -1.0, 1.0)[None, :]
    return (fwht(x) * HADAMARD_SCALE).astype(np.float32)


def hadamard_rotation32(signs) -> np.ndarray:
    """The dense fp32 matrix of the same rotation, fp32(s_i H_ij / sqrt(128)), for the parts of
    the path that take a dense R (q rotation, R_V^T)."""
    s = np.ones(D) if signs is None else np.where(np.asarray(signs) < 0, -1.0, 1.0)
    h = fwht(np.eye(D))          # row i = H e_i = row i of H (H is symmetric)
    return (s[:, None] * h * HADAMARD_SCALE).astype(np.float32)


def rotate_query(q_bits: np.ndarray, rot_k32: np.ndarray, group: int) -> np.ndarray:
    """q' = q . R_K(h) in fp64 for each query head; query head j reads KV head j // group.

    q_bits: uint16 [Hq][128]; rot_k32: float32 [Hkv][128][128].  Returns fp64 [Hq][128].
    """
    q = bf16_bits_to_f64(q_bits)
    out = np.empty_like(q)
    for j in range(q.shape[0]):
        out[j] = q[j] @ np.asarray(rot_k32[j // group], dtype=np.float32).astype(np.float64)
    return out


# ----------------------------------------------------------------------------------------
# Quantiser: per-token groups of 32 rotated channels, clipped min/max, 4 affine levels.
# ----------------------------------------------------------------------------------------

def group_params(y: np.ndarray, clip: float, levels: int = LEVELS):
    """fp16 scale and zero of every 32-channel group of every rotated row.

    For each group: mx = max, mn = min of the fp32 values (a -0.0 extreme counts as +0.0);
    the clip ratio c (as fp32) scales
    both ends, mx_c = c*mx and mn_c = c*mn in fp32; the step is s = (mx_c - mn_c) / 3 in fp32
    (3 = number of steps between 4 levels); the stored scale is fp16(s) and the stored zero
    is fp16(mn_c), both rounded to nearest even.

    y: float32 [N][128].  Returns (s16, z16) float16 [N][4].
    """
    y = np.asarray(y, dtype=np.float32)
    c = np.float32(clip)
    g = y.reshape(y.shape[0], NGROUPS, GROUP)
    # signed zeros: an extreme equal to -0.0 is taken as +0.0 (x + 0 in fp32), so the stored
    # zero's sign bit never depends on the order of a group's +0/-0 entries
    mx = (g.max(axis=2) + np.float32(0)).astype(np.float32)
    mn = (g.min(axis=2) + np.float32(0)).astype(np.float32)
    mx_c = (c * mx).astype(np.float32)
    mn_c = (c * mn).astype(np.float32)
    width = (mx_c - mn_c).astype(np.float32)
    s32 = (width / np.float32(levels - 1)).astype(np.float32)
    return s32.astype(np.float16), mn_c.astype(np.float16)


def group_codes(y: np.ndarray, s16: np.ndarray, z16: np.ndarray, levels: int = LEVELS) -> np.ndarray:
    """2-bit code of every channel: round((y - z) / s) to nearest even, clamped to [0, 3].

    The quotient uses the stored fp16 scale and zero (widened to fp32) in fp32 arithmetic, so
    the codes agree with what dequantisation reconstructs.  A group whose stored scale is 0
    gets all codes 0.

    Returns uint8 [N][128].
    """
    y = np.asarray(y, dtype=np.float32).reshape(-1, NGROUPS, GROUP)
    s = s16.astype(np.float32)[:, :, None]
    z = z16.astype(np.float32)[:, :, None]
    diff = (y - z).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        t = (diff / np.where(s == 0, np.float32(1), s)).astype(np.float32)
    code = np.clip(np.rint(t), 0, levels - 1)
    code = np.where(s == 0, 0, code)
    return code.astype(np.uint8).reshape(-1, D)


def dequant(codes: np.ndarray, s16: np.ndarray, z16: np.ndarray) -> np.ndarray:
    """Reconstructed values s*code + z in fp64 (exact). codes [N][128], s16/z16 [N][4]."""
    c = codes.astype(np.float64).reshape(-1, NGROUPS, GROUP)
    v = s16.astype(np.float64)[:, :, None] * c + z16.astype(np.float64)[:, :, None]
    return v.reshape(-1, D)


def quantize_rows(x_bits: np.ndarray, rot32, clip: float, mean32=None, hadamard_signs=None,
                  levels: int = LEVELS):
    """Rotate (after removing mean32, if given), clip and quantise rows to `levels` levels (4:
    INT2, 16: INT4): returns (y fp32, codes u8, s16, z16).  With rot32 None the rotation is the
    Hadamard one with the given signs (rotate_rows_hadamard)."""
    if rot32 is None:
        y = rotate_rows_hadamard(x_bits, hadamard_signs)
    else:
        y = rotate_rows_centered(x_bits, rot32, mean32)
    s16, z16 = group_params(y, clip, levels)
    return y, group_codes(y, s16, z16, levels), s16, z16


# ----------------------------------------------------------------------------------------
# Byte layout of one (page, KV head) INT2 record (1536 bytes).
#
#   [   0,  512)  K codes.  Channel c of page slot r: 16-channel word d = c // 16, stored as the
#                 dword at 8*(16*(d % 4) + r) + 4*(d // 4); inside the dword, byte (c % 16)//4,
#                 bits 2*(c % 4) .. +1.
#   [ 512, 1024)  V codes.  Channel c of slot r: lane chunk L = 16*(r // 4) + (c % 16) at
#                 512 + 8*L; dword (r % 4) // 2 of the chunk, 16-bit half r % 2 of the dword;
#                 inside the half, bits 2*(c // 16) .. +1.
#   [1024, 1280)  K scale/zero.  Group g of slot r: fp16 scale then fp16 zero at 1024 + 16*r + 4*g.
#   [1280, 1536)  V scale/zero, same arrangement at 1280 + 16*r + 4*g.
#
# All multi-byte fields are little-endian.
# ----------------------------------------------------------------------------------------

def k_code_location(r, c):
    """(byte offset in the record, bit offset in that byte) of K channel c of slot r.

    Works elementwise on integers or integer arrays."""
    d = c // 16
    byte = K_CODES + 8 * (16 * (d % 4) + r) + 4 * (d // 4) + (c % 16) // 4
    return byte, 2 * (c % 4)


def v_code_location(r, c):
    """(byte offset, bit offset) of V channel c of slot r; elementwise on arrays."""
    lane = 16 * (r // 4) + (c % 16)
    nb = c // 16
    byte = V_CODES + 8 * lane + 4 * ((r % 4) // 2) + 2 * (r % 2) + nb // 4
    return byte, 2 * (nb % 4)


def meta_location(kind: str, r, g):
    """Byte offset of the (fp16 scale, fp16 zero) pair of group g of slot r."""
    return (K_META if kind == "k" else V_META) + 16 * r + 4 * g


# INT4 records (the INT4 abstract on the OSCAR paper's page: token-wise INT4 in a paged
# layout).  2560 bytes per (page, KV head); 16 levels, 4 bits per code.  The arrangement of the
# codes is this implementation's own (the pages fix none), chosen for matrix-core operands:
#   [   0, 1024)  K codes in 16-byte lane chunks: chunk 16*q + r holds token slot r's channels
#                 16q .. 16q+15 (bytes 0..7) and 64+16q .. 64+16q+15 (bytes 8..15).  Channel c
#                 (h = c // 64, q = (c % 64) // 16, j = c % 16, i = j % 4) sits at byte
#                 16*(16q + r) + 8h + 4*(i // 2) + j // 4, bits 4*(i % 2): masking the chunk's
#                 dwords with 0x0F0F0F0F (shifted by 0 and 4) gives int8 vectors whose byte b of
#                 vector i is channel 16q + 4b + i, the INT2 record's operand order.
#   [1024, 2048)  V codes in 16-byte lane chunks: chunk 16*(r // 4) + (c % 16) holds channel
#                 residue c % 16 of the four token slots 4*(r // 4) .. +3.  With nb = c // 16,
#                 k = nb // 2, u = r % 4: byte 1024 + 16*chunk + 4k + 2*(u % 2) + u // 2, bits
#                 4*(nb % 2).  Each token slot owns whole bytes; a dword shifted left by 3 or
#                 right by 5 (right by 1 or 9) and masked with 0x00780078 holds column block
#                 2k's (2k + 1's) codes of tokens 0, 1 (2, 3) of the quad at the mantissa bits of
#                 two bf16 values 1 + code/16.
#   [2048, 2304)  K scale/zero: fp16 pair of group g of slot r at 2048 + 16*r + 4*g;
#   [2304, 2560)  V scale/zero, the same arrangement at 2304.
LEVELS4 = 16
RECORD4 = 2560
K4_CODES, V4_CODES, K4_META, V4_META = 0, 1024, 2048, 2304


def k4_code_location(r, c):
    """(byte offset, bit offset) of K channel c of slot r in an INT4 record; elementwise."""
    h, q, j = c // 64, (c % 64) // 16, c % 16
    i = j % 4
    return K4_CODES + 16 * (16 * q + r) + 8 * h + 4 * (i // 2) + j // 4, 4 * (i % 2)


def v4_code_location(r, c):
    """(byte offset, bit offset) of V channel c of slot r in an INT4 record; elementwise."""
    nb, u = c // 16, r % 4
    chunk = 16 * (r // 4) + c % 16
    return V4_CODES + 16 * chunk + 4 * (nb // 2) + 2 * (u % 2) + u // 2, 4 * (nb % 2)


def meta4_location(kind: str, r, g):
    return (K4_META if kind == "k" else V4_META) + 16 * r + 4 * g


_CH = np.arange(D)
_GR = np.arange(NGROUPS)


def _put_codes(flat, base, r, codes, loc, width=2):
    byte, bit = loc(r[:, None], _CH[None, :])
    idx = (base[:, None] + byte).ravel()
    bit = np.broadcast_to(bit, codes.shape).ravel().astype(np.uint8)
    mask = np.uint8((1 << width) - 1)
    np.bitwise_and.at(flat, idx, (~(mask << bit)).astype(np.uint8))
    np.bitwise_or.at(flat, idx, (codes.astype(np.uint8).ravel() << bit).astype(np.uint8))


def _get_codes(flat, base, r, loc, width=2):
    byte, bit = loc(r[:, None], _CH[None, :])
    return ((flat[base[:, None] + byte] >> np.broadcast_to(bit, byte.shape).astype(np.uint8))
            & np.uint8((1 << width) - 1)).astype(np.uint8)


def _put_meta(flat, base, r, kind, s16, z16, mloc=None):
    off = base[:, None] + (mloc or meta_location)(kind, r[:, None], _GR[None, :])
    for field, vals in ((0, s16), (2, z16)):
        u = np.asarray(vals, dtype=np.float16).view(np.uint16)
        flat[off + field] = (u & 0xFF).astype(np.uint8)
        flat[off + field + 1] = (u >> 8).astype(np.uint8)


def _get_meta(flat, base, r, kind, mloc=None):
    off = base[:, None] + (mloc or meta_location)(kind, r[:, None], _GR[None, :])
    out = []
    for field in (0, 2):
        u = flat[off + field].astype(np.uint16) | (flat[off + field + 1].astype(np.uint16) << 8)
        out.append(u.view(np.float16))
    return out[0], out[1]


def write_slots(flat, base, r, kcodes, ks16, kz16, vcodes, vs16, vz16, bits: int = 2) -> None:
    """Store n tokens' K and V encodings (in place) into a flat byte pool.

    base: int [n] byte offset of each token's record; r: int [n] page slot of each token;
    codes [n][128]; scales/zeros [n][4].  Only the bits belonging to each token's slot change.
    bits: 2 (the 1536-byte INT2 record) or 4 (the 2560-byte INT4 record).
    """
    base = np.asarray(base, dtype=np.int64)
    r = np.asarray(r, dtype=np.int64)
    if bits == 4:
        _put_codes(flat, base, r, kcodes, k4_code_location, 4)
        _put_codes(flat, base, r, vcodes, v4_code_location, 4)
        _put_meta(flat, base, r, "k", ks16, kz16, meta4_location)
        _put_meta(flat, base, r, "v", vs16, vz16, meta4_location)
        return
    _put_codes(flat, base, r, kcodes, k_code_location)
    _put_codes(flat, base, r, vcodes, v_code_location)
    _put_meta(flat, base, r, "k", ks16, kz16)
    _put_meta(flat, base, r, "v", vs16, vz16)


def read_slots(flat, base, r, bits: int = 2):
    """Decode n tokens: (kcodes, ks16, kz16, vcodes, vs16, vz16), codes [n][128], meta [n][4]."""
    base = np.asarray(base, dtype=np.int64)
    r = np.asarray(r, dtype=np.int64)
    if bits == 4:
        kc = _get_codes(flat, base, r, k4_code_location, 4)
        vc = _get_codes(flat, base, r, v4_code_location, 4)
        ks, kz = _get_meta(flat, base, r, "k", meta4_location)
        vs, vz = _get_meta(flat, base, r, "v", meta4_location)
        return kc, ks, kz, vc, vs, vz
    kc = _get_codes(flat, base, r, k_code_location)
    vc = _get_codes(flat, base, r, v_code_location)
    ks, kz = _get_meta(flat, base, r, "k")
    vs, vz = _get_meta(flat, base, r, "v")
    return kc, ks, kz, vc, vs, vz


def write_slot(record: np.ndarray, r: int, kcodes, ks16, kz16, vcodes, vs16, vz16) -> None:
    """Single-token form of write_slots on one 1536-byte record."""
    write_slots(record, [0], [r], np.asarray(kcodes)[None], np.asarray(ks16)[None],
                np.asarray(kz16)[None], np.asarray(vcodes)[None], np.asarray(vs16)[None],
                np.asarray(vz16)[None])


def read_slot(record: np.ndarray, r: int):
    """Single-token form of read_slots on one record."""
    return tuple(a[0] for a in read_slots(record, [0], [r]))


# ----------------------------------------------------------------------------------------
# Cache model: paged INT2 records + dense BF16 sink/window store.
# ----------------------------------------------------------------------------------------

def sink_window_index(pos: int, num_sink: int, window: int, new_len: int):
    """Row of the BF16 store that position `pos` goes to when the sequence length becomes
    new_len, or None.  Sinks are positions [0, S) at rows [0, S); a window position
    p >= S with p >= new_len - W goes to row S + (p mod W) (a ring)."""
    if pos < num_sink:
        return pos
    if window > 0 and pos >= new_len - window:
        return num_sink + pos % window
    return None


class Cache:
    """Oracle model of the cache a sequence batch writes.

    pages:   uint8 [num_pages][Hkv][1536]  INT2 records (bits = 4: [2560] INT4 records).
    sinkwin: uint16 [num_slots][Hkv][S+W][2][128] bf16 bits of the rotated K (index 0) and
             V (index 1) rows of sink and window positions.
    """

    def __init__(self, num_pages, num_kv_heads, num_slots, num_sink, window, fill=0, bits=2):
        self.bits = bits
        self.record = RECORD4 if bits == 4 else RECORD
        self.levels = LEVELS4 if bits == 4 else LEVELS
        self.pages = np.full((num_pages, num_kv_heads, self.record), fill, dtype=np.uint8)
        self.sinkwin = np.full((num_slots, num_kv_heads, num_sink + window, 2, D),
                               fill | (fill << 8), dtype=np.uint16)
        self.num_sink = num_sink
        self.window = window
        self.hkv = num_kv_heads

    def _bases(self, table_row, h, positions):
        pages = np.asarray(table_row)[np.asarray(positions) // PAGE].astype(np.int64)
        return (pages * self.hkv + h) * self.record, np.asarray(positions) % PAGE

    def append(self, table_row, slot, start_pos, k_bits, v_bits, rot_k32, rot_v32, clip_k, clip_v,
               k_mean32=None, hadamard_signs=None):
        """Append n new tokens of one sequence at positions start_pos .. start_pos+n-1.

        k_bits, v_bits: uint16 [n][Hkv][128] unrotated bf16 rows.  Every new position gets its
        INT2 encoding in its page record; sink positions and the last W positions of the new
        length also get bf16(y) in the BF16 store.  k_mean32 (fp32 [Hkv][128] or None): a key
        mean removed before the rotation (rotate_rows_centered).  With rot_k32 and rot_v32 None
        the rotation is the Hadamard one; hadamard_signs is then None or a pair (signs_k,
        signs_v), each None or [Hkv][128].
        """
        n = k_bits.shape[0]
        new_len = start_pos + n
        positions = np.arange(start_pos, new_len)
        flat = self.pages.reshape(-1)
        for h in range(self.hkv):
            lv = self.levels
            if rot_k32 is None:
                sk, sv = hadamard_signs if hadamard_signs is not None else (None, None)
                yk, kc, ks, kz = quantize_rows(k_bits[:, h], None, clip_k, None,
                                               None if sk is None else sk[h], lv)
                yv, vc, vs, vz = quantize_rows(v_bits[:, h], None, clip_v, None,
                                               None if sv is None else sv[h], lv)
            else:
                yk, kc, ks, kz = quantize_rows(k_bits[:, h], rot_k32[h], clip_k,
                                               None if k_mean32 is None else k_mean32[h], None, lv)
                yv, vc, vs, vz = quantize_rows(v_bits[:, h], rot_v32[h], clip_v, None, None, lv)
            base, r = self._bases(table_row, h, positions)
            write_slots(flat, base, r, kc, ks, kz, vc, vs, vz, self.bits)
            kb = f32_to_bf16_bits(yk)
            vb = f32_to_bf16_bits(yv)
            for i, pos in enumerate(positions):
                row = sink_window_index(int(pos), self.num_sink, self.window, new_len)
                if row is not None:
                    self.sinkwin[slot, h, row, 0] = kb[i]
                    self.sinkwin[slot, h, row, 1] = vb[i]

    def read_sequence(self, table_row, slot, h, length):
        """Keys and values of positions [0, length) of one KV head, in the rotated frame, fp64.

        Positions [0, min(L, S)) and the last min(W, L - n_sink) positions come from the BF16
        store; the rest is dequantised from the INT2 records.  Returns (k, v) fp64 [L][128]
        and a bool [L] mask marking the INT2 positions.
        """
        S, W = self.num_sink, self.window
        n_sink = min(length, S)
        n_win = min(W, length - n_sink)
        k = np.empty((length, D))
        v = np.empty((length, D))
        is_int2 = np.zeros(length, dtype=bool)
        for p in range(length):
            if p < n_sink:
                row = p
            elif p >= length - n_win:
                row = S + p % W
            else:
                row = None
            if row is not None:
                k[p] = bf16_bits_to_f64(self.sinkwin[slot, h, row, 0])
                v[p] = bf16_bits_to_f64(self.sinkwin[slot, h, row, 1])
            else:
                is_int2[p] = True
        idx = np.nonzero(is_int2)[0]
        if idx.size:
            kc, ks, kz, vc, vs, vz = self.decode_positions(table_row, h, idx)
            k[idx] = dequant(kc, ks, kz)
            v[idx] = dequant(vc, vs, vz)
        return k, v, is_int2

    def decode_positions(self, table_row, h, positions):
        base, r = self._bases(table_row, h, positions)
        return read_slots(self.pages.reshape(-1), base, r, self.bits)


# ----------------------------------------------------------------------------------------
# Attention.
# ----------------------------------------------------------------------------------------

def softmax_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, sm_scale: float):
    """Single-query softmax attention in fp64: returns (o [128], lse, weights [L]).

    z_p = sm * (q . k_p); a = softmax(z); o = sum_p a_p v_p; lse = max z + ln sum exp(z - max z).
    """
    z = float(np.float32(sm_scale)) * (k @ q)
    zmax = z.max()
    e = np.exp(z - zmax)
    den = e.sum()
    a = e / den
    return a @ v, zmax + np.log(den), a


def decode_attention(cache: Cache, table, slots, seq_lens, q_bits, rot_k32, rot_v32, sm_scale,
                     batches=None, heads=None):
    """Decode attention over the mixed cache, rotated frame inside, original frame out.

    q' = q . R_K(h); keys/values are the stored rotated rows (BF16 sinks/window, dequantised
    INT2 bulk); o = softmax(sm q'.k) v in the rotated frame; out = o . R_V(h)^T.

    Returns out fp64 [B][Hq][128] and lse fp64 [B][Hq] (NaN where not computed).
    """
    B, Hq = q_bits.shape[0], q_bits.shape[1]
    G = Hq // cache.hkv
    out = np.full((B, Hq, D), np.nan)
    lse = np.full((B, Hq), np.nan)
    batches = range(B) if batches is None else batches
    for b in batches:
        L = int(seq_lens[b])
        qr = rotate_query(q_bits[b], rot_k32, G)
        kv_heads = range(cache.hkv) if heads is None else sorted({j // G for j in heads})
        for h in kv_heads:
            k, v, _ = cache.read_sequence(table[b], slots[b], h, L)
            rv = np.asarray(rot_v32[h], dtype=np.float32).astype(np.float64)
            for j in range(h * G, (h + 1) * G):
                if heads is not None and j not in heads:
                    continue
                o, l, _ = softmax_attention(qr[j], k, v, sm_scale)
                out[b, j] = o @ rv.T
                lse[b, j] = l
    return out, lse


def merge_partials(m2: np.ndarray, l: np.ndarray, o: np.ndarray):
    """Merge split partials of one query row.

    Each split s carries m_s (its running max of the logits, in log2 units, i.e. logit*log2 e),
    l_s = sum of 2^(logit*log2e - m_s) and o_s = sum of 2^(...) v (unnormalised).  Splits with
    l_s == 0 are empty.  The merge is the exact softmax over the union:
        M = max_s m_s,  l = sum_s 2^(m_s - M) l_s,  o = sum_s 2^(m_s - M) o_s / l,
        lse = M ln 2 + ln l   (natural log of the sum of exp of the logits).
    m2, l: [S]; o: [S][128].  Returns (o fp64 [128], lse).
    """
    m2 = np.asarray(m2, np.float64)
    l = np.asarray(l, np.float64)
    o = np.asarray(o, np.float64)
    live = l > 0
    M = m2[live].max()
    w = np.where(live, np.exp2(np.where(live, m2, M) - M), 0.0)
    lt = (w * l).sum()
    ot = (w[:, None] * o).sum(axis=0) / lt
    return ot, M * np.log(2.0) + np.log(lt)


# ----------------------------------------------------------------------------------------
# BF16 paged baseline (no rotation, no quantisation).
#
# Page layout per (page, KV head), 8192 bytes: K as [16 tokens][128] bf16, then V transposed
# as [128 channels][16 tokens] bf16.
# ----------------------------------------------------------------------------------------

BF16_PAGE_ELEMS = 2 * PAGE * D


def bf16_write_token(page: np.ndarray, r: int, k_bits_row, v_bits_row) -> None:
    """page: uint16 [4096]; store token slot r's K row and V column."""
    page[r * D:(r + 1) * D] = k_bits_row
    page[PAGE * D + np.arange(D) * PAGE + r] = v_bits_row


def bf16_read_page(page: np.ndarray):
    k = page[:PAGE * D].reshape(PAGE, D)
    v = page[PAGE * D:].reshape(D, PAGE).T
    return k, v


def bf16_decode_attention(pages, table, seq_lens, q_bits, sm_scale, num_kv_heads):
    """Plain softmax attention over the unrotated bf16 pages. Returns out fp64 [B][Hq][128], lse."""
    B, Hq = q_bits.shape[0], q_bits.shape[1]
    G = Hq // num_kv_heads
    out = np.empty((B, Hq, D))
    lse = np.empty((B, Hq))
    for b in range(B):
        L = int(seq_lens[b])
        for h in range(num_kv_heads):
            ks = np.empty((L, D))
            vs = np.empty((L, D))
            for p0 in range(0, L, PAGE):
                kp, vp = bf16_read_page(pages[int(table[b][p0 // PAGE]), h])
                n = min(PAGE, L - p0)
                ks[p0:p0 + n] = bf16_bits_to_f64(kp[:n])
                vs[p0:p0 + n] = bf16_bits_to_f64(vp[:n])
            for j in range(h * G, (h + 1) * G):
                o, l, _ = softmax_attention(bf16_bits_to_f64(q_bits[b, j]), ks, vs, sm_scale)
                out[b, j] = o
                lse[b, j] = l
    return out, lse
