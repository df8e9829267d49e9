"""Thin ctypes binding over the C ABI in include/oscar.h.

Argument marshalling only: torch tensors (device memory owned by the caller) become raw
pointers, the current torch stream becomes the hipStream_t, and non-zero status codes become
exceptions.  Every computation runs in the HIP library; nothing here falls back to the CPU.
The library is loaded on first use and a missing build raises immediately.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("OSCAR_LIBRARY", os.path.join(_PKG, "liboscar_hip.so"))

HEAD_DIM, PAGE_SIZE, GROUP_SIZE, RECORD_BYTES = 128, 16, 32, 1536
BF16_PAGE_ELEMS = 2 * PAGE_SIZE * HEAD_DIM

EXPORTED = (
    "oscar_status_string",
    "oscar_rotate_quantize_append",
    "oscar_rotate_quantize_append_ex",
    "oscar_rotate_quantize_append_hadamard",
    "oscar_int4_rotate_quantize_append",
    "oscar_int4_decode_attention",
    "oscar_decode_workspace_bytes",
    "oscar_decode_attention",
    "oscar_combine",
    "oscar_bf16_append",
    "oscar_bf16_decode_attention",
    "oscar_read_records",
    "oscar_mfma_bf16_tiles",
    "oscar_decode_attention_static",
    "oscar_prepare_queries",
    "oscar_decode_attention_prepared",
    "oscar_append_and_prepare",
)

STATIC_WORKSPACE_BYTES = 32 << 20   # OSCAR_STATIC_WORKSPACE_BYTES
# Partial slots per (sequence, query head) that follow the max_splits INT2 slots in a decode
# workspace: the BF16 sink/window parts (include/oscar.h, oscar_decode_workspace_bytes).
WINDOW_SLOTS = 8


class OscarError(RuntimeError):
    def __init__(self, fn: str, code: int, msg: str):
        super().__init__(f"{fn} failed with status {code}: {msg}")
        self.code = code


class Layout(ctypes.Structure):
    _fields_ = [
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("group_size", ctypes.c_int32),
        ("num_sink", ctypes.c_int32),
        ("window", ctypes.c_int32),
        ("num_pages", ctypes.c_int32),
        ("max_pages_per_seq", ctypes.c_int32),
        ("num_slots", ctypes.c_int32),
    ]


def make_layout(num_kv_heads, num_sink, window, num_pages, max_pages_per_seq, num_slots,
                head_dim=HEAD_DIM, page_size=PAGE_SIZE, group_size=GROUP_SIZE) -> Layout:
    return Layout(num_kv_heads, head_dim, page_size, group_size, num_sink, window, num_pages,
                  max_pages_per_seq, num_slots)


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load liboscar_hip.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"HIP library not built: {path} is missing "
                           "(run python -m int2_rotated_kv_rotate_amd.build)")
    lib = ctypes.CDLL(path)
    P, I32, F32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    LP = ctypes.POINTER(Layout)
    lib.oscar_status_string.argtypes = [I32]
    lib.oscar_status_string.restype = ctypes.c_char_p
    lib.oscar_rotate_quantize_append.argtypes = [LP, P, P, P, P, I32, I32, P, P, P, P, P, P, F32, F32, P]
    lib.oscar_rotate_quantize_append.restype = I32
    lib.oscar_rotate_quantize_append_ex.argtypes = [LP, P, P, P, P, I32, I32, P, P, P, P, P, P, P,
                                                    F32, F32, I32, P]
    lib.oscar_rotate_quantize_append_ex.restype = I32
    lib.oscar_rotate_quantize_append_hadamard.argtypes = [LP, P, P, P, P, I32, I32, P, P, P, P, P, P,
                                                          F32, F32, P]
    lib.oscar_rotate_quantize_append_hadamard.restype = I32
    lib.oscar_int4_rotate_quantize_append.argtypes = [LP, P, P, P, P, I32, I32, P, P, P, P, P, P, P,
                                                      F32, F32, P]
    lib.oscar_int4_rotate_quantize_append.restype = I32
    lib.oscar_int4_decode_attention.argtypes = [LP, P, P, P, P, I32, I32, P, P, P, F32, I32, I32,
                                                P, SZ, P]
    lib.oscar_int4_decode_attention.restype = I32
    lib.oscar_decode_workspace_bytes.argtypes = [I32, I32, I32]
    lib.oscar_decode_workspace_bytes.restype = SZ
    lib.oscar_decode_attention.argtypes = [LP, P, P, P, P, I32, I32, P, P, P, F32, I32, I32, P, SZ, P]
    lib.oscar_decode_attention.restype = I32
    lib.oscar_prepare_queries.argtypes = [LP, I32, I32, P, P, P, I32, I32, P, SZ, P]
    lib.oscar_prepare_queries.restype = I32
    lib.oscar_append_and_prepare.argtypes = [LP, P, P, P, P, I32, I32, P, P, P, P, P, P, P, F32,
                                             F32, I32, P, P, I32, I32, P, SZ, P]
    lib.oscar_append_and_prepare.restype = I32
    lib.oscar_decode_attention_prepared.argtypes = [LP, P, P, P, P, I32, I32, P, F32, I32, I32, P,
                                                    SZ, P]
    lib.oscar_decode_attention_prepared.restype = I32
    lib.oscar_combine.argtypes = [I32, I32, I32, I32, P, SZ, P, P, P, P]
    lib.oscar_combine.restype = I32
    lib.oscar_bf16_append.argtypes = [LP, P, P, I32, I32, P, P, P, P, P]
    lib.oscar_bf16_append.restype = I32
    lib.oscar_bf16_decode_attention.argtypes = [LP, P, P, I32, I32, P, P, F32, I32, I32, P, SZ, P]
    lib.oscar_bf16_decode_attention.restype = I32
    lib.oscar_decode_attention_static.argtypes = [LP, P, P, P, P, I32, I32, P, P, P, P, F32, I32,
                                                  I32, P, P, P]
    lib.oscar_decode_attention_static.restype = I32
    lib.oscar_read_records.argtypes = [P, I32, P, I32, I32, P, P]
    lib.oscar_mfma_bf16_tiles.argtypes = [P, P, P, P, I32, P]
    lib.oscar_mfma_bf16_tiles.restype = I32
    lib.oscar_read_records.restype = I32
    _lib = lib
    return lib


def _check(fn: str, code: int) -> None:
    if code != 0:
        msg = load_library().oscar_status_string(code).decode()
        raise OscarError(fn, code, msg)


def _ptr(t: Optional[torch.Tensor], dtype=None, name: str = "") -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name}: expected a GPU tensor")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: expected a contiguous tensor")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


# Append kernels (include/oscar.h OSCAR_APPEND_*): all write the same bytes.
APPEND_AUTO, APPEND_VECTOR, APPEND_MATRIX = 0, 1, 2


def rotate_quantize_append(lay: Layout, pages, sinkwin, block_table, slot_ids, k_new, v_new,
                           new_offsets, start_pos, rot_k, rot_v, clip_k: float, clip_v: float,
                           stream=None, method: int = APPEND_AUTO, k_mean=None) -> None:
    """pages uint8 [P][Hkv][1536]; sinkwin int16 bf16 bits [slots][Hkv][S+W][2][128];
    k_new/v_new int16 bf16 bits [N][Hkv][128]; new_offsets int32 [B+1]; start_pos int32 [B];
    rot_k/rot_v float32 [Hkv][128][128].  method: APPEND_AUTO, APPEND_VECTOR or APPEND_MATRIX.
    k_mean: None or float32 [Hkv][128], a key mean removed before the key rotation."""
    lib = load_library()
    batch = start_pos.numel()
    _check("oscar_rotate_quantize_append_ex", lib.oscar_rotate_quantize_append_ex(
        ctypes.byref(lay), _ptr(pages, torch.uint8, "pages"), _ptr(sinkwin, torch.int16, "sinkwin"),
        _ptr(block_table, torch.int32, "block_table"), _ptr(slot_ids, torch.int32, "slot_ids"),
        batch, k_new.shape[0], _ptr(k_new, torch.int16, "k_new"), _ptr(v_new, torch.int16, "v_new"),
        _ptr(new_offsets, torch.int32, "new_offsets"), _ptr(start_pos, torch.int32, "start_pos"),
        _ptr(rot_k, torch.float32, "rot_k"), _ptr(rot_v, torch.float32, "rot_v"),
        _ptr(k_mean, torch.float32, "k_mean"), float(clip_k), float(clip_v), int(method),
        _stream(stream)))


def rotate_quantize_append_hadamard(lay: Layout, pages, sinkwin, block_table, slot_ids, k_new,
                                    v_new, new_offsets, start_pos, signs_k, signs_v,
                                    clip_k: float, clip_v: float, stream=None) -> None:
    """As rotate_quantize_append with the Hadamard rotation diag(s) H / sqrt(128) for K and V;
    signs_k / signs_v: None or int8 [Hkv][128]."""
    lib = load_library()
    batch = start_pos.numel()
    _check("oscar_rotate_quantize_append_hadamard", lib.oscar_rotate_quantize_append_hadamard(
        ctypes.byref(lay), _ptr(pages, torch.uint8, "pages"), _ptr(sinkwin, torch.int16, "sinkwin"),
        _ptr(block_table, torch.int32, "block_table"), _ptr(slot_ids, torch.int32, "slot_ids"),
        batch, k_new.shape[0], _ptr(k_new, torch.int16, "k_new"), _ptr(v_new, torch.int16, "v_new"),
        _ptr(new_offsets, torch.int32, "new_offsets"), _ptr(start_pos, torch.int32, "start_pos"),
        _ptr(signs_k, torch.int8, "signs_k"), _ptr(signs_v, torch.int8, "signs_v"),
        float(clip_k), float(clip_v), _stream(stream)))


INT4_RECORD_BYTES = 2560


def int4_rotate_quantize_append(lay: Layout, pages, sinkwin, block_table, slot_ids, k_new, v_new,
                                new_offsets, start_pos, rot_k, rot_v, clip_k: float,
                                clip_v: float, stream=None, k_mean=None) -> None:
    """As rotate_quantize_append into an INT4 pool uint8 [P][Hkv][2560]."""
    lib = load_library()
    batch = start_pos.numel()
    _check("oscar_int4_rotate_quantize_append", lib.oscar_int4_rotate_quantize_append(
        ctypes.byref(lay), _ptr(pages, torch.uint8, "pages"), _ptr(sinkwin, torch.int16, "sinkwin"),
        _ptr(block_table, torch.int32, "block_table"), _ptr(slot_ids, torch.int32, "slot_ids"),
        batch, k_new.shape[0], _ptr(k_new, torch.int16, "k_new"), _ptr(v_new, torch.int16, "v_new"),
        _ptr(new_offsets, torch.int32, "new_offsets"), _ptr(start_pos, torch.int32, "start_pos"),
        _ptr(rot_k, torch.float32, "rot_k"), _ptr(rot_v, torch.float32, "rot_v"),
        _ptr(k_mean, torch.float32, "k_mean"), float(clip_k), float(clip_v), _stream(stream)))


def int4_decode_attention(lay: Layout, pages, sinkwin, block_table, slot_ids, q, seq_lens, rot_k,
                          sm_scale: float, split_pages: int, max_splits: int, workspace,
                          stream=None) -> None:
    """Decode attention over an INT4 pool; finish with combine()."""
    lib = load_library()
    batch, hq = q.shape[0], q.shape[1]
    _check("oscar_int4_decode_attention", lib.oscar_int4_decode_attention(
        ctypes.byref(lay), _ptr(pages, torch.uint8, "pages"), _ptr(sinkwin, torch.int16, "sinkwin"),
        _ptr(block_table, torch.int32, "block_table"), _ptr(slot_ids, torch.int32, "slot_ids"),
        batch, hq, _ptr(q, torch.int16, "q"), _ptr(seq_lens, torch.int32, "seq_lens"),
        _ptr(rot_k, torch.float32, "rot_k"), float(sm_scale), int(split_pages), int(max_splits),
        _ptr(workspace, torch.uint8, "workspace"), workspace.numel(), _stream(stream)))


def decode_workspace_bytes(batch: int, num_q_heads: int, max_splits: int) -> int:
    return int(load_library().oscar_decode_workspace_bytes(batch, num_q_heads, max_splits))


def decode_attention(lay: Layout, pages, sinkwin, block_table, slot_ids, q, seq_lens, rot_k,
                     sm_scale: float, num_workers: int, max_splits: int, workspace,
                     stream=None) -> None:
    """num_workers: worker wavefronts (0 = one per resident slot of the device)."""
    lib = load_library()
    batch, hq = q.shape[0], q.shape[1]
    _check("oscar_decode_attention", lib.oscar_decode_attention(
        ctypes.byref(lay), _ptr(pages, torch.uint8, "pages"), _ptr(sinkwin, torch.int16, "sinkwin"),
        _ptr(block_table, torch.int32, "block_table"), _ptr(slot_ids, torch.int32, "slot_ids"),
        batch, hq, _ptr(q, torch.int16, "q"), _ptr(seq_lens, torch.int32, "seq_lens"),
        _ptr(rot_k, torch.float32, "rot_k"), float(sm_scale), num_workers, max_splits,
        _ptr(workspace, torch.uint8, "workspace"), workspace.numel(), _stream(stream)))


def prepare_queries(lay: Layout, q, seq_lens, rot_k, num_workers: int, max_splits: int,
                    workspace, stream=None) -> None:
    """First half of decode_attention: q' and the work plan into the workspace."""
    lib = load_library()
    batch, hq = q.shape[0], q.shape[1]
    _check("oscar_prepare_queries", lib.oscar_prepare_queries(
        ctypes.byref(lay), batch, hq, _ptr(q, torch.int16, "q"),
        _ptr(seq_lens, torch.int32, "seq_lens"), _ptr(rot_k, torch.float32, "rot_k"),
        num_workers, max_splits, _ptr(workspace, torch.uint8, "workspace"), workspace.numel(),
        _stream(stream)))


def append_and_prepare(lay: Layout, pages, sinkwin, block_table, slot_ids, k_new, v_new,
                       new_offsets, start_pos, rot_k, rot_v, clip_k: float, clip_v: float, q,
                       seq_lens, num_workers: int, max_splits: int, workspace, k_mean=None,
                       stream=None) -> None:
    """rotate_quantize_append (APPEND_AUTO) of this step's new rows and prepare_queries of the
    same batch in one call (one launch below 256 new rows); batch = start_pos.numel() =
    q.shape[0]."""
    lib = load_library()
    batch, hq = q.shape[0], q.shape[1]
    if start_pos.numel() != batch:
        raise ValueError("append_and_prepare: start_pos and q disagree on the batch")
    _check("oscar_append_and_prepare", lib.oscar_append_and_prepare(
        ctypes.byref(lay), _ptr(pages, torch.uint8, "pages"), _ptr(sinkwin, torch.int16, "sinkwin"),
        _ptr(block_table, torch.int32, "block_table"), _ptr(slot_ids, torch.int32, "slot_ids"),
        batch, k_new.shape[0], _ptr(k_new, torch.int16, "k_new"), _ptr(v_new, torch.int16, "v_new"),
        _ptr(new_offsets, torch.int32, "new_offsets"), _ptr(start_pos, torch.int32, "start_pos"),
        _ptr(rot_k, torch.float32, "rot_k"), _ptr(rot_v, torch.float32, "rot_v"),
        _ptr(k_mean, torch.float32, "k_mean"), float(clip_k), float(clip_v), hq,
        _ptr(q, torch.int16, "q"), _ptr(seq_lens, torch.int32, "seq_lens"), num_workers,
        max_splits, _ptr(workspace, torch.uint8, "workspace"), workspace.numel(), _stream(stream)))


def decode_attention_prepared(lay: Layout, pages, sinkwin, block_table, slot_ids, batch: int,
                              num_q_heads: int, seq_lens, sm_scale: float, num_workers: int,
                              max_splits: int, workspace, stream=None) -> None:
    """Second half of decode_attention, from a workspace filled by prepare_queries."""
    lib = load_library()
    _check("oscar_decode_attention_prepared", lib.oscar_decode_attention_prepared(
        ctypes.byref(lay), _ptr(pages, torch.uint8, "pages"), _ptr(sinkwin, torch.int16, "sinkwin"),
        _ptr(block_table, torch.int32, "block_table"), _ptr(slot_ids, torch.int32, "slot_ids"),
        batch, num_q_heads, _ptr(seq_lens, torch.int32, "seq_lens"), float(sm_scale), num_workers,
        max_splits, _ptr(workspace, torch.uint8, "workspace"), workspace.numel(), _stream(stream)))


def decode_attention_static(lay: Layout, pages, sinkwin, block_table, slot_ids, q, seq_lens,
                            rot_k, rot_v, sm_scale: float, num_workers: int, max_splits: int,
                            out, lse=None, stream=None) -> None:
    """Decode attention + combine with the library's own workspace (no allocation)."""
    lib = load_library()
    batch, hq = q.shape[0], q.shape[1]
    _check("oscar_decode_attention_static", lib.oscar_decode_attention_static(
        ctypes.byref(lay), _ptr(pages, torch.uint8, "pages"), _ptr(sinkwin, torch.int16, "sinkwin"),
        _ptr(block_table, torch.int32, "block_table"), _ptr(slot_ids, torch.int32, "slot_ids"),
        batch, hq, _ptr(q, torch.int16, "q"), _ptr(seq_lens, torch.int32, "seq_lens"),
        _ptr(rot_k, torch.float32, "rot_k"), _ptr(rot_v, torch.float32, "rot_v"),
        float(sm_scale), num_workers, max_splits, _ptr(out, torch.float32, "out"),
        _ptr(lse, torch.float32, "lse"), _stream(stream)))


def combine(batch: int, num_q_heads: int, num_kv_heads: int, max_splits: int, workspace,
            rot_v, out, lse=None, stream=None) -> None:
    lib = load_library()
    _check("oscar_combine", lib.oscar_combine(
        batch, num_q_heads, num_kv_heads, max_splits, _ptr(workspace, torch.uint8, "workspace"),
        workspace.numel(), _ptr(rot_v, torch.float32, "rot_v"), _ptr(out, torch.float32, "out"),
        _ptr(lse, torch.float32, "lse"), _stream(stream)))


def bf16_append(lay: Layout, pages, block_table, k_new, v_new, new_offsets, start_pos,
                stream=None) -> None:
    lib = load_library()
    _check("oscar_bf16_append", lib.oscar_bf16_append(
        ctypes.byref(lay), _ptr(pages, torch.int16, "pages"),
        _ptr(block_table, torch.int32, "block_table"), start_pos.numel(), k_new.shape[0],
        _ptr(k_new, torch.int16, "k_new"), _ptr(v_new, torch.int16, "v_new"),
        _ptr(new_offsets, torch.int32, "new_offsets"), _ptr(start_pos, torch.int32, "start_pos"),
        _stream(stream)))


def bf16_decode_attention(lay: Layout, pages, block_table, q, seq_lens, sm_scale: float,
                          split_pages: int, max_splits: int, workspace, stream=None) -> None:
    lib = load_library()
    batch, hq = q.shape[0], q.shape[1]
    _check("oscar_bf16_decode_attention", lib.oscar_bf16_decode_attention(
        ctypes.byref(lay), _ptr(pages, torch.int16, "pages"),
        _ptr(block_table, torch.int32, "block_table"), batch, hq, _ptr(q, torch.int16, "q"),
        _ptr(seq_lens, torch.int32, "seq_lens"), float(sm_scale), split_pages, max_splits,
        _ptr(workspace, torch.uint8, "workspace"), workspace.numel(), _stream(stream)))


def read_records(pages, record_ids, num_workers: int, out, stream=None) -> None:
    """Read-bandwidth probe: reads the INT2 records record_ids (page * Hkv + head) of the pool
    with the decode kernel's access pattern and writes per-lane XORs to out (uint32 / int32
    [64 * num_workers])."""
    lib = load_library()
    if out.numel() < 64 * num_workers:
        raise ValueError("out: needs 64 * num_workers entries")
    _check("oscar_read_records", lib.oscar_read_records(
        _ptr(pages, torch.uint8, "pages"), pages.numel() // RECORD_BYTES,
        _ptr(record_ids, torch.int32, "record_ids"),
        record_ids.numel(), num_workers, _ptr(out, torch.int32, "out"), _stream(stream)))


def mfma_bf16_tiles(a, b, c, d, stream=None) -> None:
    """D = A . B + C per 16x16x32 tile with one bf16 matrix-core instruction: a int16 (bf16 bits)
    [tiles][16][32], b [tiles][32][16], c and d float32 [tiles][16][16]."""
    lib = load_library()
    tiles = a.shape[0]
    if a.shape != (tiles, 16, 32) or b.shape != (tiles, 32, 16) or c.shape != (tiles, 16, 16) \
            or d.shape != (tiles, 16, 16):
        raise ValueError("mfma_bf16_tiles: shapes [T][16][32], [T][32][16], [T][16][16] x 2")
    _check("oscar_mfma_bf16_tiles", lib.oscar_mfma_bf16_tiles(
        _ptr(a, torch.int16, "a"), _ptr(b, torch.int16, "b"), _ptr(c, torch.float32, "c"),
        _ptr(d, torch.float32, "d"), tiles, _stream(stream)))
