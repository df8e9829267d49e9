"""Device-side driver for the library: caches in HBM, seeded inputs, one decode step.

Plumbing only (torch for device memory and streams); every step of the method runs in the
HIP library through ``ops``.  Used by the tests, the smoke check and the benchmark.
"""
from __future__ import annotations

import dataclasses
import math
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Optional, Sequence

import numpy as np
import torch

from . import ops
from . import workload as W

SM_SCALE = float(np.float32(1.0 / math.sqrt(128.0)))


@dataclasses.dataclass
class Problem:
    """Host-side description of one decode step on a workload (numpy arrays)."""
    w: W.Workload
    lens: np.ndarray            # int64 [B], context length including the decoded token
    table: np.ndarray           # int32 [B][max_pages]
    num_pages: int
    rot_k: np.ndarray           # float32 [Hkv][128][128]
    rot_v: np.ndarray
    q: np.ndarray               # uint16 bf16 bits [B][Hq][128]

    @property
    def batch(self):
        return self.w.batch


def make_problem(w: W.Workload, lens: Optional[Sequence[int]] = None, extra_pages: int = 3,
                 rot_k: Optional[np.ndarray] = None, rot_v: Optional[np.ndarray] = None) -> Problem:
    lens = W.seq_lengths(w) if lens is None else np.asarray(lens, dtype=np.int64)
    table, num_pages = W.block_table(w, lens, extra_pages=extra_pages)
    rk = (W.rotations(w, "k") if rot_k is None else rot_k).astype(np.float32)
    rv = (W.rotations(w, "v") if rot_v is None else rot_v).astype(np.float32)
    return Problem(w, lens, table, num_pages, rk, rv, W.queries(w))


def as_i16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16))


class GpuCache:
    """INT2 page pool + BF16 sink/window store + block table on the GPU."""

    def __init__(self, p: Problem, device="cuda", fill: Optional[int] = None,
                 k_mean: Optional[np.ndarray] = None, hadamard_signs=None, bits: int = 2):
        """k_mean: None or fp32 [Hkv][128], a key mean removed before the key rotation on every
        append into this cache.  hadamard_signs: None for the dense rotations p.rot_k / p.rot_v,
        else a pair (signs_k, signs_v) (each None or int8 [Hkv][128]) for appends with the
        Hadamard rotation; p.rot_k / p.rot_v must then be its dense form (attention reads them).
        bits: 2 (INT2 records) or 4 (the INT4 variant, 2560-byte records)."""
        w = p.w
        self.p = p
        self.device = device
        self.layout = ops.make_layout(w.num_kv_heads, w.num_sink, w.window, p.num_pages,
                                      p.table.shape[1], w.batch)
        self.bits = bits
        rec = ops.INT4_RECORD_BYTES if bits == 4 else ops.RECORD_BYTES
        self.pages = torch.empty((p.num_pages, w.num_kv_heads, rec), dtype=torch.uint8,
                                 device=device)
        self.sinkwin = torch.empty((w.batch, w.num_kv_heads, max(w.num_sink + w.window, 1), 2, 128),
                                   dtype=torch.int16, device=device)
        if fill is not None:
            self.pages.fill_(fill)
            v16 = fill | (fill << 8)
            self.sinkwin.fill_(v16 - 65536 if v16 >= 32768 else v16)
        self.table = torch.from_numpy(p.table).to(device)
        self.slots = torch.arange(w.batch, dtype=torch.int32, device=device)
        self.rot_k = torch.from_numpy(p.rot_k).to(device)
        self.rot_v = torch.from_numpy(p.rot_v).to(device)
        self.k_mean = (None if k_mean is None else
                       torch.from_numpy(np.ascontiguousarray(k_mean, dtype=np.float32)).to(device))
        self.hadamard = hadamard_signs is not None
        self.signs = tuple(None if sg is None else
                           torch.from_numpy(np.ascontiguousarray(sg, dtype=np.int8)).to(device)
                           for sg in (hadamard_signs or (None, None)))

    def append(self, k_rows: Sequence[np.ndarray], v_rows: Sequence[np.ndarray],
               start: Sequence[int], method: int = ops.APPEND_AUTO):
        """Append rows for every sequence b (bf16 bits [n_b][Hkv][128], n_b may be 0) at
        positions start[b], start[b]+1, ...  Lists are indexed by sequence."""
        counts = np.array([r.shape[0] for r in k_rows], dtype=np.int64)
        if counts.sum() == 0:
            return
        offs = np.zeros(len(k_rows) + 1, dtype=np.int32)
        offs[1:] = np.cumsum(counts)
        k = as_i16(np.concatenate(k_rows)).to(self.device)
        v = as_i16(np.concatenate(v_rows)).to(self.device)
        if self.bits == 4:
            ops.int4_rotate_quantize_append(
                self.layout, self.pages, self.sinkwin, self.table, self.slots, k, v,
                torch.from_numpy(offs).to(self.device),
                torch.from_numpy(np.asarray(start, dtype=np.int32)).to(self.device),
                self.rot_k, self.rot_v, self.p.w.clip, self.p.w.clip, k_mean=self.k_mean)
            return
        if self.hadamard:
            ops.rotate_quantize_append_hadamard(
                self.layout, self.pages, self.sinkwin, self.table, self.slots, k, v,
                torch.from_numpy(offs).to(self.device),
                torch.from_numpy(np.asarray(start, dtype=np.int32)).to(self.device),
                self.signs[0], self.signs[1], self.p.w.clip, self.p.w.clip)
            return
        ops.rotate_quantize_append(
            self.layout, self.pages, self.sinkwin, self.table, self.slots, k, v,
            torch.from_numpy(offs).to(self.device),
            torch.from_numpy(np.asarray(start, dtype=np.int32)).to(self.device),
            self.rot_k, self.rot_v, self.p.w.clip, self.p.w.clip, method=method,
            k_mean=self.k_mean)

    def fill_context(self, chunk_tokens: int = 1 << 20, keep_tail: int = 0):
        """Append positions [0, L_b - 1) of every sequence (everything but the decoded token),
        in chunks of whole sequences.  Returns the per-sequence last rows (k, v) [1][Hkv][128];
        with keep_tail > 0 also the rows of positions [L_b - 1 - keep_tail, L_b - 1)."""
        w = self.p.w
        hkv = w.num_kv_heads
        empty = np.zeros((0, hkv, 128), dtype=np.uint16)
        needle = W.needle_site(w, self.p.lens)
        offsets, outliers = W.key_offsets(w), W.outlier_channels(w)
        last_k, last_v, tail_k, tail_v = [], [], [], []
        pend_k = [empty] * w.batch
        pend_v = [empty] * w.batch
        pend_n = 0

        def gen(b):
            return W.sequence_kv(w, b, int(self.p.lens[b]), offsets=offsets, outliers=outliers,
                                 needle=needle, q_bits=self.p.q)

        workers = max(1, min(16, os.cpu_count() or 1))
        with ThreadPoolExecutor(workers) as ex:
            for g0 in range(0, w.batch, 2 * workers):
                group = list(range(g0, min(w.batch, g0 + 2 * workers)))
                for b, (kb, vb) in zip(group, ex.map(gen, group)):
                    L = int(self.p.lens[b])
                    last_k.append(kb[L - 1:L])
                    last_v.append(vb[L - 1:L])
                    if keep_tail:
                        t0 = max(0, L - 1 - keep_tail)
                        tail_k.append(kb[t0:L - 1].copy())
                        tail_v.append(vb[t0:L - 1].copy())
                    pend_k[b] = kb[:L - 1]
                    pend_v[b] = vb[:L - 1]
                    pend_n += L - 1
                    if pend_n >= chunk_tokens or b == w.batch - 1:
                        self.append(pend_k, pend_v, [0] * w.batch)
                        torch.cuda.synchronize()
                        pend_k = [empty] * w.batch
                        pend_v = [empty] * w.batch
                        pend_n = 0
        if keep_tail:
            return last_k, last_v, tail_k, tail_v
        return last_k, last_v


# Partial slots per (sequence, KV head): enough that the run length is set by the worker count
# for the contexts used here (a pair of P pages needs about P / run + 1 slots).
DEFAULT_MAX_SPLITS = 64
MAX_SPLITS_CAP = 512
SMALL_LAUNCH_PAIRS = 128   # (sequence, KV head) pairs below which runs are cut short
SHORT_RUN_PAGES = 16      # run length aimed at for such launches (fastest decode + combine
                          # at Qwen3-4B 32K and 128K, batch 1)


def default_max_splits(batch: int, num_kv_heads: int, max_context: int) -> int:
    """Slots per (sequence, KV head) for a decode launch.  With many pairs the worker count
    sets the run length and DEFAULT_MAX_SPLITS is ample; with few pairs (batch 1) the runs are
    cut to about SHORT_RUN_PAGES pages so that a long context spreads over the device, at most
    MAX_SPLITS_CAP slots."""
    if batch * num_kv_heads >= SMALL_LAUNCH_PAIRS:
        return DEFAULT_MAX_SPLITS
    pages = -(-max(1, max_context) // 16)
    want = -(-pages // SHORT_RUN_PAGES) + 2
    return int(min(MAX_SPLITS_CAP, max(DEFAULT_MAX_SPLITS, want)))


class DecodeStep:
    """Buffers and launches of one decode step: append the new token, attend, combine."""

    def __init__(self, cache: GpuCache, num_workers: int = 0, max_splits: Optional[int] = None,
                 ws_fill: Optional[int] = None):
        """num_workers 0: one worker per resident wavefront slot; max_splits bounds the INT2
        partials per (sequence, KV head) (a small value lengthens the workers' runs); None
        takes default_max_splits.  ws_fill: a byte written over the whole workspace first
        (0xFF makes every float in it a NaN; the kernels must not depend on its contents)."""
        p = cache.p
        self.cache = cache
        self.num_workers = num_workers
        self.max_splits = (max_splits if max_splits is not None
                           else default_max_splits(p.batch, p.w.num_kv_heads, int(p.lens.max())))
        if cache.bits == 4:   # INT4: fixed page splits, about 8192 workgroups over the batch
            pages_max = -(-int(p.lens.max()) // 16)
            self.split_pages = max(1, -(-pages_max * p.batch * p.w.num_kv_heads // 8192))
            if max_splits is None:
                self.max_splits = max(1, -(-pages_max // self.split_pages))
        dev = cache.device
        self.ws = torch.empty(ops.decode_workspace_bytes(p.batch, p.w.num_q_heads, self.max_splits),
                              dtype=torch.uint8, device=dev)
        if ws_fill is not None:
            self.ws.fill_(ws_fill)
        self.q = as_i16(p.q).to(dev)
        self.seq_lens = torch.from_numpy(p.lens.astype(np.int32)).to(dev)
        self.out = torch.empty((p.batch, p.w.num_q_heads, 128), dtype=torch.float32, device=dev)
        self.lse = torch.empty((p.batch, p.w.num_q_heads), dtype=torch.float32, device=dev)
        self.new_off = torch.arange(p.batch + 1, dtype=torch.int32, device=dev)
        self.start = torch.from_numpy((p.lens - 1).astype(np.int32)).to(dev)
        self.k_last = None
        self.v_last = None
        self.side = None            # second stream of run_overlapped, made on first use

    def set_new_token(self, last_k, last_v):
        self.k_last = as_i16(np.concatenate(last_k)).to(self.cache.device)
        self.v_last = as_i16(np.concatenate(last_v)).to(self.cache.device)

    def append_new(self, stream=None):
        c = self.cache
        if c.bits == 4:
            ops.int4_rotate_quantize_append(c.layout, c.pages, c.sinkwin, c.table, c.slots,
                                            self.k_last, self.v_last, self.new_off, self.start,
                                            c.rot_k, c.rot_v, c.p.w.clip, c.p.w.clip, stream,
                                            k_mean=c.k_mean)
            return
        if c.hadamard:
            ops.rotate_quantize_append_hadamard(c.layout, c.pages, c.sinkwin, c.table, c.slots,
                                                self.k_last, self.v_last, self.new_off, self.start,
                                                c.signs[0], c.signs[1], c.p.w.clip, c.p.w.clip,
                                                stream)
            return
        ops.rotate_quantize_append(c.layout, c.pages, c.sinkwin, c.table, c.slots, self.k_last,
                                   self.v_last, self.new_off, self.start, c.rot_k, c.rot_v,
                                   c.p.w.clip, c.p.w.clip, stream, k_mean=c.k_mean)

    def decode_only(self, stream=None):
        c = self.cache
        if c.bits == 4:
            ops.int4_decode_attention(c.layout, c.pages, c.sinkwin, c.table, c.slots, self.q,
                                      self.seq_lens, c.rot_k, SM_SCALE, self.split_pages,
                                      self.max_splits, self.ws, stream)
            return
        ops.decode_attention(c.layout, c.pages, c.sinkwin, c.table, c.slots, self.q, self.seq_lens,
                             c.rot_k, SM_SCALE, self.num_workers, self.max_splits, self.ws, stream)

    def combine_only(self, stream=None):
        c = self.cache
        p = c.p
        ops.combine(p.batch, p.w.num_q_heads, p.w.num_kv_heads, self.max_splits, self.ws, c.rot_v,
                    self.out, self.lse, stream)

    def attend(self, stream=None):
        self.decode_only(stream)
        self.combine_only(stream)

    def run(self, stream=None):
        self.append_new(stream)
        self.attend(stream)

    # The step with the decode split in two, on one stream (run_split) or with the new token's
    # append on a second stream overlapped with the query preparation (run_overlapped: the two
    # are independent; the decode waits for both).  INT2 caches only.
    def prepare(self, stream=None):
        c = self.cache
        ops.prepare_queries(c.layout, self.q, self.seq_lens, c.rot_k, self.num_workers,
                            self.max_splits, self.ws, stream)

    def decode_prepared(self, stream=None):
        c = self.cache
        p = c.p
        ops.decode_attention_prepared(c.layout, c.pages, c.sinkwin, c.table, c.slots, p.batch,
                                      p.w.num_q_heads, self.seq_lens, SM_SCALE, self.num_workers,
                                      self.max_splits, self.ws, stream)

    def run_split(self, before_decode=None, after_decode=None):
        """The step through the two halves of the decode on the current stream: append,
        prepare, decode, combine (the same kernels as run()).  before_decode() and
        after_decode(), if given, run right before and after the decode kernel's launch."""
        self.append_new()
        self.prepare()
        if before_decode is not None:
            before_decode()
        self.decode_prepared()
        if after_decode is not None:
            after_decode()
        self.combine_only()

    def append_and_prepare(self, stream=None):
        c = self.cache
        ops.append_and_prepare(c.layout, c.pages, c.sinkwin, c.table, c.slots, self.k_last,
                               self.v_last, self.new_off, self.start, c.rot_k, c.rot_v,
                               c.p.w.clip, c.p.w.clip, self.q, self.seq_lens, self.num_workers,
                               self.max_splits, self.ws, k_mean=c.k_mean, stream=stream)

    def run_fused(self, before_decode=None, after_decode=None):
        """The step with the append and the query preparation in one call
        (oscar_append_and_prepare), then decode and combine, on the current stream; the same
        bytes as run_split().  INT2 caches with a dense rotation only."""
        c = self.cache
        if c.bits != 2 or c.hadamard:
            raise ValueError("run_fused: INT2 caches with a dense rotation only")
        self.append_and_prepare()
        if before_decode is not None:
            before_decode()
        self.decode_prepared()
        if after_decode is not None:
            after_decode()
        self.combine_only()

    def run_overlapped(self, before_decode=None, after_decode=None):
        """append || prepare, then decode and combine on the current stream.  before_decode()
        and after_decode(), if given, run on the current stream right before and after the
        decode kernel's launch (event markers)."""
        main = torch.cuda.current_stream()
        if self.side is None:
            self.side = torch.cuda.Stream()      # default priority
        side = self.side
        side.wait_stream(main)      # the previous step's decode has read the pool
        with torch.cuda.stream(side):
            self.append_new(side)
        self.prepare(main)
        main.wait_stream(side)
        if before_decode is not None:
            before_decode()
        self.decode_prepared(main)
        if after_decode is not None:
            after_decode()
        self.combine_only(main)


def capture_graph(fn) -> "torch.cuda.CUDAGraph":
    """A HIP graph of the launches fn issues on the current stream: replay() re-issues them with
    the same buffers and arguments, without the host's per-launch work in between.  fn runs
    once eagerly on a side stream first, so that the library's one-time queries (compute-unit
    count, occupancy) happen outside the capture.  The library's launch paths record kernels
    only (no memset or copy nodes)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


class Bf16Cache:
    """Device buffers of the BF16 paged baseline for a Problem (no rotation, no quantisation):
    pages int16 [num_pages][Hkv][4096] (bf16 K [16][128] then V^T [128][16]) filled with every
    sequence's whole context, plus a decode workspace split every `split_pages` pages."""

    def __init__(self, p: Problem, device="cuda", split_pages: Optional[int] = None):
        w = p.w
        self.p = p
        self.device = device
        hkv = w.num_kv_heads
        self.layout = ops.make_layout(hkv, 0, 0, p.num_pages, p.table.shape[1], w.batch)
        self.pages = torch.zeros((p.num_pages, hkv, ops.BF16_PAGE_ELEMS), dtype=torch.int16,
                                 device=device)
        self.table = torch.from_numpy(p.table).to(device)
        offsets, outliers = W.key_offsets(w), W.outlier_channels(w)
        for b in range(w.batch):
            L = int(p.lens[b])
            kb, vb = W.sequence_kv(w, b, L, offsets=offsets, outliers=outliers)
            ops.bf16_append(self.layout, self.pages, self.table[b:b + 1],
                            as_i16(kb).to(device), as_i16(vb).to(device),
                            torch.tensor([0, L], dtype=torch.int32, device=device),
                            torch.zeros(1, dtype=torch.int32, device=device))
        torch.cuda.synchronize()
        pages_max = int((p.lens.max() + 15) // 16)
        if split_pages is None:  # about 1024 (split, KV head, sequence) waves: one per SIMD
            split_pages = max(1, -(-pages_max * w.batch * hkv // 1024))
        self.split_pages = split_pages
        self.max_splits = max(1, -(-pages_max // split_pages))
        self.ws = torch.empty(ops.decode_workspace_bytes(w.batch, w.num_q_heads, self.max_splits),
                              dtype=torch.uint8, device=device)
        self.q = as_i16(p.q).to(device)
        self.seq_lens = torch.from_numpy(p.lens.astype(np.int32)).to(device)
        self.out = torch.empty((w.batch, w.num_q_heads, 128), dtype=torch.float32, device=device)
        self.lse = torch.empty((w.batch, w.num_q_heads), dtype=torch.float32, device=device)

    def attend(self, stream=None):
        w = self.p.w
        ops.bf16_decode_attention(self.layout, self.pages, self.table, self.q, self.seq_lens,
                                  SM_SCALE, self.split_pages, self.max_splits, self.ws, stream)
        ops.combine(w.batch, w.num_q_heads, w.num_kv_heads, self.max_splits, self.ws, None,
                    self.out, self.lse, stream)
