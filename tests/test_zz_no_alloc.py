"""oscar_decode_attention_static (decode attention + combine with the library's own device
workspace, for callers that cannot allocate) against oscar_decode_attention + oscar_combine on a
caller-allocated workspace: the same bits, on two calls in a row, the second with a smaller
input (the buffer then holds the first call's contents); a request larger than the buffer is
refused before anything is launched."""
import sys

import numpy as np
import pytest
import torch

from oracle import oscar_oracle as O
from int2_rotated_kv_rotate_amd import harness as H
from int2_rotated_kv_rotate_amd import ops
from int2_rotated_kv_rotate_amd import workload as W

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, file=sys.stderr, flush=True)


def _case(name, base, **over):
    w = W.scaled(base, name=name, **over)
    p = H.make_problem(w)
    cache = H.GpuCache(p, fill=0xA5)
    last_k, last_v = cache.fill_context()
    step = H.DecodeStep(cache, num_workers=0, max_splits=16, ws_fill=0xFF)
    step.set_new_token(last_k, last_v)
    step.run()          # append + decode_attention + combine on the torch-allocated workspace
    torch.cuda.synchronize()
    return p, cache, step


def _static(cache, step):
    p = cache.p
    out = torch.full_like(step.out, float("nan"))
    lse = torch.full_like(step.lse, float("nan"))
    ops.decode_attention_static(cache.layout, cache.pages, cache.sinkwin, cache.table,
                                cache.slots, step.q, step.seq_lens, cache.rot_k, cache.rot_v,
                                H.SM_SCALE, step.num_workers, step.max_splits, out, lse)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


def test_static_workspace_matches_allocated_workspace():
    cases = [("static_big", W.WORKLOADS["qwen3_8b_b64"], dict(batch=6, ctx=2600, ctx_min=900)),
             ("static_small", W.WORKLOADS["qwen3_4b"], dict(batch=2, ctx=700, ctx_min=300))]
    for name, base, over in cases:
        p, cache, step = _case(name, base, **over)
        need = ops.decode_workspace_bytes(p.batch, p.w.num_q_heads, step.max_splits)
        _log(f"[no-alloc] {name}: B={p.batch} lens={p.lens.tolist()} workspace {need} bytes")
        assert need <= ops.STATIC_WORKSPACE_BYTES
        out, lse = _static(cache, step)
        ref_out, ref_lse = step.out.cpu().numpy(), step.lse.cpu().numpy()
        assert np.array_equal(out, ref_out), f"{name}: out differs from the allocated-workspace path"
        assert np.array_equal(lse, ref_lse), f"{name}: lse differs from the allocated-workspace path"
        if name == "static_small":   # and the oracle, to the attention tolerance
            oc = O.Cache(p.num_pages, p.w.num_kv_heads, p.batch, p.w.num_sink, p.w.window,
                         fill=0xA5)
            needle = W.needle_site(p.w, p.lens)
            for b in range(p.batch):
                L = int(p.lens[b])
                kb, vb = W.sequence_kv(p.w, b, L, needle=needle, q_bits=p.q)
                oc.append(p.table[b], b, 0, kb[:L - 1], vb[:L - 1], p.rot_k, p.rot_v, p.w.clip,
                          p.w.clip)
                oc.append(p.table[b], b, L - 1, kb[L - 1:], vb[L - 1:], p.rot_k, p.rot_v,
                          p.w.clip, p.w.clip)
            ref, ref_l = O.decode_attention(oc, p.table, np.arange(p.batch), p.lens, p.q,
                                            p.rot_k, p.rot_v, H.SM_SCALE)
            rel = np.abs(out - ref).max(-1) / np.abs(ref).max(-1)
            assert rel.max() <= 2e-3 and np.abs(lse - ref_l).max() <= 2e-3
        del step, cache


def test_static_workspace_refuses_oversized_requests():
    w = W.scaled(W.WORKLOADS["qwen3_4b"], name="static_refuse", batch=2, ctx=300)
    p = H.make_problem(w)
    cache = H.GpuCache(p)
    step = H.DecodeStep(cache, max_splits=8)
    too_many = 1500   # 2 x 32 query heads x 1508 slots x 520 bytes > 32 MiB
    assert ops.decode_workspace_bytes(2, w.num_q_heads, too_many) > ops.STATIC_WORKSPACE_BYTES
    sentinel = torch.full_like(step.out, 7.0)
    with pytest.raises(ops.OscarError) as e:
        ops.decode_attention_static(cache.layout, cache.pages, cache.sinkwin, cache.table,
                                    cache.slots, step.q, step.seq_lens, cache.rot_k, cache.rot_v,
                                    H.SM_SCALE, 0, too_many, sentinel)
    assert e.value.code == 3
    torch.cuda.synchronize()
    assert torch.all(sentinel == 7.0)    # nothing was launched
