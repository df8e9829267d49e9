"""The decode step split in two (oscar_prepare_queries, then oscar_decode_attention_prepared)
with the new token's append on a second stream gives the one-stream step's results bit for bit.

The append and the query preparation are independent, so a serving loop overlaps them and joins
before the decode.  Each case runs the one-stream step (append, oscar_decode_attention,
oscar_combine), keeps its outputs and cache, then runs the overlapped step several times with
the outputs NaN-filled in between: every run must reproduce the outputs exactly and leave the
page pool and sink/window store byte-identical (the append rewrites the same bytes).
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
    "b40_ragged": ("qwen3_8b_b64", dict(batch=40, ctx=900, ctx_min=200)),
    "g8_b2": ("qwen3_32b", dict(batch=2, ctx=900)),
}


@pytest.mark.parametrize("name", list(CASES))
def test_overlapped_step_matches_one_stream_step(name):
    wname, over = CASES[name]
    w = W.scaled(W.WORKLOADS[wname], **over)
    print(f"[overlap] {name}: B={w.batch} heads {w.num_q_heads}/{w.num_kv_heads}", file=sys.stderr,
          flush=True)
    p = H.make_problem(w)
    cache = H.GpuCache(p)
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
        step.run_overlapped()
        torch.cuda.synchronize()
        assert torch.equal(step.out, out0), f"{name}: run {rep}: out differs"
        assert torch.equal(step.lse, lse0), f"{name}: run {rep}: lse differs"
        assert torch.equal(cache.pages, pages0), f"{name}: run {rep}: page pool changed"
        assert torch.equal(cache.sinkwin, sw0), f"{name}: run {rep}: sink/window store changed"
    assert np.isfinite(out0.cpu().numpy()).all()
