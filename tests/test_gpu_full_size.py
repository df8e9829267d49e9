"""GPU parity at full workload sizes, in the launch configuration bench.py times.

Qwen3-8B layer shape, batch 64, context lengths uniform in [16384, 32768] (the benchmark
workload, 4 query heads per KV head); Qwen3-32B layer shape, batch 16, context 32768 (8 query
heads per KV head, the other row layout of the decode kernel); and Qwen3-4B layer shape, batch
1, context 32768 (the small-launch path: sink/window workgroups first, one q-rotation workgroup
per query head, short worker runs, the per-query-head combine); and the Qwen3-8B batch-64
workload with INT4 records (the matrix-core INT4 decode); sink 4 + window 128 in BF16,
INT2 (or INT4) bulk, one worker wavefront per resident slot (num_workers = 0) and the harness's default
partial-slot count (64 at large batch, enough for ~24-page runs at batch 1).  Both sides start from pools filled with a 0xA5 sentinel; the decode
workspace starts filled with 0xFF bytes.

The whole batch runs on the GPU; the oracle recomputes sampled (sequence, KV head) pairs one by
one (the shortest and the longest sequence and one in between, on different KV heads):
  * every page record of the pair's sequence and its sink/window rows must be byte-identical,
  * the pair's G output rows must be within 2e-3 per row (max abs error / max abs reference),
    its lse within 2e-3;
and every output row of the batch must be finite.
"""
import math
import sys

import numpy as np
import pytest
import torch

from oracle import oscar_oracle as O
from int2_rotated_kv_rotate_amd import harness as H
from int2_rotated_kv_rotate_amd import workload as W

pytestmark = pytest.mark.gpu

TOL = 2e-3
SENTINEL = 0xA5


def _log(msg):
    print(msg, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", params=["qwen3_8b_b64", "qwen3_32b", "qwen3_4b", "qwen3_8b_b64_int4"])
def full_run(request):
    bits = 4 if request.param.endswith("_int4") else 2
    w = W.WORKLOADS[request.param.removesuffix("_int4")]
    _log(f"[full] workload {w.name}: batch {w.batch}, {w.num_q_heads}/{w.num_kv_heads} heads, "
         f"INT{bits}")
    p = H.make_problem(w)
    cache = H.GpuCache(p, fill=SENTINEL, bits=bits)
    last_k, last_v = cache.fill_context()
    step = H.DecodeStep(cache, ws_fill=0xFF)          # bench.py's configuration: auto workers, 64 slots
    step.set_new_token(last_k, last_v)
    step.run()
    torch.cuda.synchronize()
    return w, p, cache, step, bits


def _oracle_pair(w, p, b, h, bits):
    """Oracle cache of one (sequence, KV head) built by the same appends as the GPU run
    (context, then the decoded token), and its decode attention for the G query heads."""
    L = int(p.lens[b])
    G = w.group
    kb, vb = W.sequence_kv(w, b, L, offsets=W.key_offsets(w), outliers=W.outlier_channels(w),
                           needle=W.needle_site(w, p.lens), q_bits=p.q)
    oc = O.Cache(p.num_pages, 1, w.batch, w.num_sink, w.window, fill=SENTINEL, bits=bits)
    args = (p.rot_k[h:h + 1], p.rot_v[h:h + 1], w.clip, w.clip)
    oc.append(p.table[b], b, 0, kb[:L - 1, h:h + 1], vb[:L - 1, h:h + 1], *args)
    oc.append(p.table[b], b, L - 1, kb[L - 1:, h:h + 1], vb[L - 1:, h:h + 1], *args)
    ref, ref_lse = O.decode_attention(oc, p.table[b:b + 1], np.array([b]), p.lens[b:b + 1],
                                      p.q[b:b + 1, h * G:(h + 1) * G], p.rot_k[h:h + 1],
                                      p.rot_v[h:h + 1], H.SM_SCALE)
    return oc, ref[0], ref_lse[0]


def test_full_size_outputs_finite(full_run):
    _, _, _, step, _ = full_run
    assert torch.isfinite(step.out).all()
    assert torch.isfinite(step.lse).all()


@pytest.mark.parametrize("which,h", [("shortest", 0), ("middle", 3), ("longest", 7)])
def test_full_size_sampled_pairs(full_run, which, h):
    w, p, cache, step, bits = full_run
    order = np.argsort(p.lens, kind="stable")
    b = int({"shortest": order[0], "middle": order[len(order) // 2], "longest": order[-1]}[which])
    L = int(p.lens[b])
    G = w.group
    _log(f"[full] {which}: sequence {b} L={L} KV head {h}")
    oc, ref, ref_lse = _oracle_pair(w, p, b, h, bits)

    pages_b = p.table[b, :math.ceil(L / 16)]
    gpu_rec = cache.pages[torch.from_numpy(pages_b.astype(np.int64)).to(cache.pages.device), h]
    gpu_rec = gpu_rec.cpu().numpy()
    mism = np.nonzero(gpu_rec != oc.pages[pages_b, 0])
    assert mism[0].size == 0, f"{mism[0].size} record bytes differ"
    sw = cache.sinkwin[b, h].cpu().numpy().view(np.uint16)
    assert np.array_equal(sw, oc.sinkwin[b, 0]), "sink/window rows differ"

    out = step.out[b, h * G:(h + 1) * G].cpu().numpy().astype(np.float64)
    lse = step.lse[b, h * G:(h + 1) * G].cpu().numpy().astype(np.float64)
    rel = np.abs(out - ref).max(axis=-1) / np.abs(ref).max(axis=-1)
    # elementwise, relative to max(|ref|, a quarter of the row's largest |ref|)
    el = np.abs(out - ref) / np.maximum(np.abs(ref), 0.25 * np.abs(ref).max(-1, keepdims=True))
    _log(f"[full] {which}: max row rel err {rel.max():.3e}, max elementwise {el.max():.3e}, "
         f"max |dlse| {np.abs(lse - ref_lse).max():.3e}")
    assert rel.max() <= TOL
    assert el.max() <= TOL
    assert np.abs(lse - ref_lse).max() <= TOL
