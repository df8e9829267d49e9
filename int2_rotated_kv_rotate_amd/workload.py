"""Seeded synthetic workloads for the rotated-INT2 KV cache and its decode attention.

This module only draws inputs. It holds none of the method's arithmetic (no rotation of
cache rows, no quantisation, no attention), so the CPU oracle and the HIP library can both
be fed from it without sharing any of the computation they are compared on.

Shapes follow the Qwen3-style layers the OSCAR pages evaluate on (OSCAR paper abstract,
thelatestinai.com/papers/2605.17757, "Abstract": Qwen3-4B/8B/32B, reasoning traces up to 32k
tokens, needle retrieval up to 128K).  The pages' datasets and trained weights are not
available, so every tensor is synthetic:

* q and V are N(0, 1); K is N(0, 1) plus a per-(KV head, channel) offset drawn from
  N(0, variance 2), and 4 seeded outlier channels per KV head are scaled by 15.  Every value
  is rounded to bf16 (round to nearest, ties to even) before use.
* The fixed rotation of each KV head is the Q factor of a QR decomposition of a seeded
  128 x 128 N(0, 1) matrix (stand-in for the offline calibrated rotation).
* The block table maps each sequence's logical pages to a seeded random permutation of the
  physical pages of the pool.

Every stream is derived from one SeedSequence per workload, spawned in a fixed order, and K/V
are drawn per sequence so one sequence can be regenerated without the rest of the batch.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

HEAD_DIM = 128
PAGE_SIZE = 16
GROUP_SIZE = 32
RECORD_BYTES = 1536  # one (page, KV head) INT2 record
BF16_PAGE_BYTES = 2 * PAGE_SIZE * HEAD_DIM * 2  # one (page, KV head) BF16 K+V page

# Child stream order under each workload's root SeedSequence.
_STREAMS = ("rot_k", "rot_v", "q", "k", "v", "offsets", "outliers", "lengths", "block_table", "needle")


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    ctx: int                      # context length (max when ragged)
    ctx_min: Optional[int]        # ragged lengths uniform in [ctx_min, ctx] when set
    num_sink: int
    window: int
    clip: float
    seed: int
    prefill_new: int = 0          # tokens appended per sequence by the prefill-append step
    needle: bool = False
    needle_scale: float = 8.0     # the planted key is needle_scale * q / |q| of its query head
    bf16_batches: tuple = ()      # batches of the BF16 paged baseline at equal KV memory

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads


WORKLOADS = {
    "tiny": Workload("tiny", 1, 1, 1, 512, None, 4, 64, 0.95, 1000),
    "qwen3_4b": Workload("qwen3_4b", 1, 32, 8, 32768, None, 4, 128, 0.95, 1001),
    "qwen3_8b_b64": Workload("qwen3_8b_b64", 64, 32, 8, 32768, 16384, 4, 128, 0.95, 1002,
                             prefill_new=2048),
    "qwen3_32b": Workload("qwen3_32b", 16, 64, 8, 32768, None, 4, 128, 0.95, 1003,
                          bf16_batches=(2, 3)),
    "long_128k": Workload("long_128k", 1, 32, 8, 131072, None, 4, 128, 0.95, 1004, needle=True),
}


def scaled(w: Workload, *, batch=None, ctx=None, ctx_min=None, name=None) -> Workload:
    """A smaller copy of a workload with the same head structure, seeds and distributions.

    ctx_min=None keeps fixed lengths; pass it to keep ragged lengths in [ctx_min, ctx].
    """
    return dataclasses.replace(
        w, batch=w.batch if batch is None else batch, ctx=w.ctx if ctx is None else ctx,
        ctx_min=ctx_min, name=name or (w.name + "_scaled"))


def _streams(w: Workload) -> dict:
    root = np.random.SeedSequence(w.seed)
    return dict(zip(_STREAMS, root.spawn(len(_STREAMS))))


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); returns the uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    u = u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
    return (u >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def rotations(w: Workload, which: str = "k") -> np.ndarray:
    """fp64 [Hkv][128][128] orthogonal matrices, one per KV head (row-vector use: y = x @ R)."""
    ss = _streams(w)["rot_k" if which == "k" else "rot_v"]
    rng = np.random.default_rng(ss)
    out = np.empty((w.num_kv_heads, HEAD_DIM, HEAD_DIM), dtype=np.float64)
    for h in range(w.num_kv_heads):
        a = rng.standard_normal((HEAD_DIM, HEAD_DIM))
        q, _ = np.linalg.qr(a)
        out[h] = q
    return out


def seq_lengths(w: Workload) -> np.ndarray:
    """int64 [B] context lengths (including the token decoded this step)."""
    if w.ctx_min is None:
        return np.full(w.batch, w.ctx, dtype=np.int64)
    rng = np.random.default_rng(_streams(w)["lengths"])
    return rng.integers(w.ctx_min, w.ctx, size=w.batch, endpoint=True).astype(np.int64)


def block_table(w: Workload, lens: np.ndarray, extra_pages: int = 0):
    """Seeded random-permutation block table.

    Returns (table int32 [B][max_pages], num_pages).  Unused entries are -1.  `extra_pages`
    appends unused physical pages to the pool (so a pool can be larger than the cache).
    """
    pages_per_seq = (np.asarray(lens) + PAGE_SIZE - 1) // PAGE_SIZE
    total = int(pages_per_seq.sum())
    num_pages = total + extra_pages
    rng = np.random.default_rng(_streams(w)["block_table"])
    perm = rng.permutation(num_pages)[:total].astype(np.int32)
    max_pages = int(pages_per_seq.max())
    table = np.full((len(lens), max_pages), -1, dtype=np.int32)
    o = 0
    for b, n in enumerate(pages_per_seq):
        table[b, :n] = perm[o:o + n]
        o += n
    return table, num_pages


def queries(w: Workload) -> np.ndarray:
    """bf16 bits [B][Hq][128], N(0, 1)."""
    rng = np.random.default_rng(_streams(w)["q"])
    return to_bf16_bits(rng.standard_normal((w.batch, w.num_q_heads, HEAD_DIM), dtype=np.float32))


def key_offsets(w: Workload) -> np.ndarray:
    rng = np.random.default_rng(_streams(w)["offsets"])
    return (rng.standard_normal((w.num_kv_heads, HEAD_DIM)) * math.sqrt(2.0)).astype(np.float32)


def outlier_channels(w: Workload) -> np.ndarray:
    rng = np.random.default_rng(_streams(w)["outliers"])
    return np.stack([np.sort(rng.choice(HEAD_DIM, size=4, replace=False))
                     for _ in range(w.num_kv_heads)]).astype(np.int64)


def key_channel_means(w: Workload) -> np.ndarray:
    """fp32 [Hkv][128]: the mean of the generated keys per (KV head, channel), i.e. the channel
    offset, times 15 on the outlier channels (the keys are (N(0,1) + offset) * scale)."""
    mu = key_offsets(w).astype(np.float32).copy()
    out = outlier_channels(w)
    for h in range(w.num_kv_heads):
        mu[h, out[h]] *= np.float32(15.0)
    return mu


def needle_site(w: Workload, lens: np.ndarray):
    """(b, position, kv_head, query_head) of the planted needle, or None."""
    if not w.needle:
        return None
    rng = np.random.default_rng(_streams(w)["needle"])
    h = int(rng.integers(0, w.num_kv_heads))
    j = h * w.group + int(rng.integers(0, w.group))
    return 0, int(lens[0]) // 2, h, j


def sequence_kv(w: Workload, b: int, length: int, *, offsets=None, outliers=None,
                needle=None, q_bits=None):
    """Unrotated bf16 bits K, V of sequence b: each [length][Hkv][128] uint16.

    Deterministic in (workload, b) and independent of the rest of the batch.  Positions are
    drawn as a prefix of a fixed-length stream, so a shorter `length` gives a prefix of the
    same sequence.
    """
    st = _streams(w)
    kss = st["k"].spawn(w.batch)[b]
    vss = st["v"].spawn(w.batch)[b]
    if offsets is None:
        offsets = key_offsets(w)
    if outliers is None:
        outliers = outlier_channels(w)
    krng = np.random.default_rng(kss)
    vrng = np.random.default_rng(vss)
    k = krng.standard_normal((length, w.num_kv_heads, HEAD_DIM), dtype=np.float32)
    k += offsets[None]
    for h in range(w.num_kv_heads):
        k[:, h, outliers[h]] *= np.float32(15.0)
    v = vrng.standard_normal((length, w.num_kv_heads, HEAD_DIM), dtype=np.float32)
    kb = to_bf16_bits(k)
    vb = to_bf16_bits(v)
    if needle is not None and needle[0] == b and needle[1] < length:
        _, p, h, j = needle
        qv = bf16_bits_to_f32(q_bits[b, j]).astype(np.float64)
        kb[p, h] = to_bf16_bits((w.needle_scale * qv / np.linalg.norm(qv)).astype(np.float32))
    return kb, vb


def synthetic_partials(seed: int, batch: int, num_q_heads: int, num_slots: int, valid: np.ndarray):
    """Random split partials (m in log2 units, l > 0, o') for testing the split merge alone.

    valid: bool [B][num_slots]; invalid slots get m = -inf, l = 0, o' = 0.
    """
    rng = np.random.default_rng(seed)
    m = (rng.standard_normal((batch, num_q_heads, num_slots)) * 4.0).astype(np.float32)
    l = rng.uniform(0.5, 40.0, (batch, num_q_heads, num_slots)).astype(np.float32)
    o = rng.standard_normal((batch, num_q_heads, num_slots, HEAD_DIM)).astype(np.float32)
    vmask = np.broadcast_to(np.asarray(valid)[:, None, :], m.shape)
    m = np.where(vmask, m, -np.inf).astype(np.float32)
    l = np.where(vmask, l, 0.0).astype(np.float32)
    o = np.where(vmask[..., None], o, 0.0).astype(np.float32)
    return m, l, o
