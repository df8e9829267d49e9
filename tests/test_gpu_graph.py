"""HIP-graph replay of the decode step gives the eager step's results bit for bit.

A serving loop at batch 1 captures the step (append the new token, decode attention, combine)
in a graph, because there the kernels finish before the host has issued the next launch.  The
graph must re-issue exactly the eager launches: the same kernels, arguments and buffers, no
memset or copy nodes.  Each case captures the step once and replays it three times, with the
program's own eager work between the replays (an eager step, outputs overwritten with NaN,
synchronisations); every replay must reproduce the eager outputs exactly, and the page pool
and sink/window store must be unchanged by the replays (the append rewrites the same bytes).
"""
import sys

import numpy as np
import pytest
import torch

from int2_rotated_kv_rotate_amd import harness as H
from int2_rotated_kv_rotate_amd import workload as W

pytestmark = pytest.mark.gpu

CASES = {
    # name: (workload, overrides)
    "b1_32_8": ("qwen3_4b", dict(batch=1, ctx=1500)),
    "b3_ragged": ("qwen3_8b_b64", dict(batch=3, ctx=1200, ctx_min=300)),
    "g8_b2": ("qwen3_32b", dict(batch=2, ctx=900)),
}


def _log(msg):
    print(msg, file=sys.stderr, flush=True)


@pytest.mark.parametrize("name", list(CASES))
def test_graph_replay_matches_eager_step(name):
    wname, over = CASES[name]
    w = W.scaled(W.WORKLOADS[wname], **over)
    _log(f"[graph] {name}: B={w.batch} heads {w.num_q_heads}/{w.num_kv_heads} ctx {w.ctx}")
    p = H.make_problem(w)
    cache = H.GpuCache(p)
    last_k, last_v = cache.fill_context()
    step = H.DecodeStep(cache)
    step.set_new_token(last_k, last_v)
    step.run()
    torch.cuda.synchronize()
    out0, lse0 = step.out.clone(), step.lse.clone()
    pages0, sw0 = cache.pages.clone(), cache.sinkwin.clone()

    g = H.capture_graph(step.run)
    for rep in range(3):
        step.run()                       # eager work between replays
        step.out.fill_(float("nan"))
        step.lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(step.out, out0), f"{name}: replay {rep}: out differs from eager"
        assert torch.equal(step.lse, lse0), f"{name}: replay {rep}: lse differs from eager"
        assert torch.equal(cache.pages, pages0), f"{name}: replay {rep}: page pool changed"
        assert torch.equal(cache.sinkwin, sw0), f"{name}: replay {rep}: sink/window store changed"
    assert np.isfinite(out0.cpu().numpy()).all()


def test_graph_replay_bf16_baseline():
    w = W.scaled(W.WORKLOADS["qwen3_4b"], batch=2, ctx=1000, ctx_min=400)
    p = H.make_problem(w)
    bc = H.Bf16Cache(p)
    bc.attend()
    torch.cuda.synchronize()
    out0, lse0 = bc.out.clone(), bc.lse.clone()
    g = H.capture_graph(bc.attend)
    for rep in range(3):
        bc.attend()
        bc.out.fill_(float("nan"))
        bc.lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(bc.out, out0), f"replay {rep}: out differs from eager"
        assert torch.equal(bc.lse, lse0), f"replay {rep}: lse differs from eager"
