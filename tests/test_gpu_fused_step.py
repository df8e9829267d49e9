"""oscar_append_and_prepare (the new rows' append and the query preparation in one launch) writes
the bytes of the two separate calls, and the decode step through it gives the usual step's
results bit for bit.

Each step case runs the usual step (append, oscar_decode_attention, oscar_combine), keeps its
outputs and cache, then runs the fused step (oscar_append_and_prepare,
oscar_decode_attention_prepared, oscar_combine) several times with the outputs NaN-filled in
between: every run must reproduce the outputs exactly and leave the page pool and sink/window
store byte-identical.  The cases cover the small-launch preparation (batch 1: one workgroup per
query head), a ragged batch, G = 8 and a key mean on the append.  A multi-token append (320 rows,
past the 4-row vector kernel) takes the two-launch branch and is compared with the two calls.
"""
import sys

import numpy as np
import pytest
import torch

from int2_rotated_kv_rotate_amd import harness as H
from int2_rotated_kv_rotate_amd import ops
from int2_rotated_kv_rotate_amd import workload as W

pytestmark = pytest.mark.gpu

CASES = {
    # name: (workload, overrides, key mean)
    "b1_32_8": ("qwen3_4b", dict(batch=1, ctx=1500), False),
    "b40_ragged": ("qwen3_8b_b64", dict(batch=40, ctx=900, ctx_min=200), False),
    "g8_b2": ("qwen3_32b", dict(batch=2, ctx=900), False),
    "b6_key_mean": ("qwen3_8b_b64", dict(batch=6, ctx=700, ctx_min=300), True),
}


@pytest.mark.parametrize("name", list(CASES))
def test_fused_step_matches_usual_step(name):
    wname, over, with_mean = CASES[name]
    w = W.scaled(W.WORKLOADS[wname], **over)
    print(f"[fused] {name}: B={w.batch} heads {w.num_q_heads}/{w.num_kv_heads} "
          f"key mean {with_mean}", file=sys.stderr, flush=True)
    p = H.make_problem(w)
    cache = H.GpuCache(p, k_mean=W.key_channel_means(w) if with_mean else None)
    last_k, last_v = cache.fill_context()
    step = H.DecodeStep(cache)
    step.set_new_token(last_k, last_v)
    step.run()
    torch.cuda.synchronize()
    out0, lse0 = step.out.clone(), step.lse.clone()
    pages0, sw0 = cache.pages.clone(), cache.sinkwin.clone()
    for rep in range(3):
        step.out.fill_(float("nan"))
        step.lse.fill_(float("nan"))
        step.run_fused()
        torch.cuda.synchronize()
        assert torch.equal(step.out, out0), f"{name}: run {rep}: out differs"
        assert torch.equal(step.lse, lse0), f"{name}: run {rep}: lse differs"
        assert torch.equal(cache.pages, pages0), f"{name}: run {rep}: page pool changed"
        assert torch.equal(cache.sinkwin, sw0), f"{name}: run {rep}: sink/window store changed"
    assert np.isfinite(out0.cpu().numpy()).all()


def test_multi_token_append_takes_two_launches_with_the_same_bytes():
    w = W.scaled(W.WORKLOADS["qwen3_8b_b64"], batch=8, ctx=600, ctx_min=400)
    tail = 40                                   # 8 x 40 = 320 new rows >= 256
    p = H.make_problem(w)
    caches = []
    for _ in range(2):
        cache = H.GpuCache(p, fill=0xA5)
        _, _, tail_k, tail_v = cache.fill_context(keep_tail=tail)
        caches.append(cache)
    offs = np.zeros(w.batch + 1, dtype=np.int32)
    offs[1:] = np.cumsum([t.shape[0] for t in tail_k])
    assert offs[-1] >= 256
    kt = H.as_i16(np.concatenate(tail_k)).cuda()
    vt = H.as_i16(np.concatenate(tail_v)).cuda()
    offs_d = torch.from_numpy(offs).cuda()
    # the tail rows take positions L-1-tail .. L-2 (position L-1 is the step's decode token)
    start_d = torch.from_numpy((p.lens - 1 - tail).astype(np.int32)).cuda()
    q = torch.from_numpy(p.q.view(np.int16)).cuda()
    lens = torch.from_numpy((p.lens - 1).astype(np.int32)).cuda()
    max_splits = 16
    nbytes = ops.decode_workspace_bytes(w.batch, w.num_q_heads, max_splits)
    ws = [torch.full((nbytes,), 0x5A, dtype=torch.uint8, device="cuda") for _ in range(2)]
    a, b = caches
    ops.rotate_quantize_append(a.layout, a.pages, a.sinkwin, a.table, a.slots, kt, vt, offs_d,
                               start_d, a.rot_k, a.rot_v, w.clip, w.clip)
    ops.prepare_queries(a.layout, q, lens, a.rot_k, 0, max_splits, ws[0])
    ops.append_and_prepare(b.layout, b.pages, b.sinkwin, b.table, b.slots, kt, vt, offs_d, start_d,
                           b.rot_k, b.rot_v, w.clip, w.clip, q, lens, 0, max_splits, ws[1])
    torch.cuda.synchronize()
    assert torch.equal(a.pages, b.pages), "page pools differ"
    assert torch.equal(a.sinkwin, b.sinkwin), "sink/window stores differ"
    assert torch.equal(ws[0], ws[1]), "workspaces (q blocks and plan) differ"
