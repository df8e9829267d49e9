"""GPU parity of the INT4 variant against the CPU oracle (bits = 4).

* Append: INT4 page pools (2560-byte records) and sink/window stores, pre-filled with a 0xA5
  sentinel on both sides, equal byte for byte after the same appends (plain and with a key mean).
* Decode: oscar_int4_decode_attention + oscar_combine within 2e-3 normwise per (sequence, query
  head) row of the oracle's decode of the same INT4 cache, lse within 2e-3; cases span G = 1,
  2, 4 and 8 (the matrix-core kernel in both row layouts), ragged lengths, a context entirely in
  BF16, a single token, a budget of two partials per (sequence, KV head), and a key whose logit
  jumps ~170 binades past the run's reference (the exact-max recomputation).
* The INT4 output is closer to exact attention over the unquantised keys and values than the
  INT2 output of the same inputs.
"""
import dataclasses
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


def _oracle_cache(p, k_mean=None):
    w = p.w
    oc = O.Cache(p.num_pages, w.num_kv_heads, w.batch, w.num_sink, w.window, fill=SENTINEL, bits=4)
    needle = W.needle_site(w, p.lens)
    for b in range(w.batch):
        L = int(p.lens[b])
        kb, vb = W.sequence_kv(w, b, L, needle=needle, q_bits=p.q)
        oc.append(p.table[b], b, 0, kb[:L - 1], vb[:L - 1], p.rot_k, p.rot_v, w.clip, w.clip, k_mean)
        oc.append(p.table[b], b, L - 1, kb[L - 1:], vb[L - 1:], p.rot_k, p.rot_v, w.clip, w.clip,
                  k_mean)
    return oc


def _run(p, max_splits=None, k_mean=None, bits=4):
    cache = H.GpuCache(p, fill=SENTINEL, k_mean=k_mean, bits=bits)
    lk, lv = cache.fill_context()
    step = H.DecodeStep(cache, ws_fill=0xFF, max_splits=max_splits)
    step.set_new_token(lk, lv)
    step.run()
    torch.cuda.synchronize()
    return cache, step


def _row_err(gpu, ref):
    return np.abs(gpu.astype(np.float64) - ref).max(axis=-1) / np.maximum(np.abs(ref).max(axis=-1), 1e-30)


CASES = {
    "tiny": (W.WORKLOADS["tiny"], {}, None),
    "q4b_ragged": (W.WORKLOADS["qwen3_4b"], dict(batch=3, ctx=1500, ctx_min=300), None),
    "q32b_g8": (W.WORKLOADS["qwen3_32b"], dict(batch=2, ctx=900), None),
    "q32b_g8_ragged": (W.WORKLOADS["qwen3_32b"], dict(batch=3, ctx=1400, ctx_min=300), None),
    "q32b_g8_few_splits": (W.WORKLOADS["qwen3_32b"], dict(batch=2, ctx=1200, ctx_min=900), 2),
    "q32b_g8_spike": (dataclasses.replace(W.WORKLOADS["qwen3_32b"], needle=True, needle_scale=128.0),
                      dict(batch=2, ctx=1200, ctx_min=900), None),
    "all_bf16": (W.WORKLOADS["tiny"], dict(ctx=60), None),
    "one_token": (W.WORKLOADS["qwen3_4b"], dict(batch=1, ctx=1), None),
    "few_splits": (W.WORKLOADS["qwen3_8b_b64"], dict(batch=2, ctx=1200, ctx_min=900), 2),
    "g2_no_sink_window16": (dataclasses.replace(W.WORKLOADS["qwen3_4b"], num_q_heads=16, num_sink=0,
                                                window=16), dict(batch=2, ctx=800, ctx_min=500), None),
    # a key of 128 q/|q| mid-sequence: one token lane's running max jumps by ~170 binades
    "spike": (dataclasses.replace(W.WORKLOADS["qwen3_4b"], needle=True, needle_scale=128.0),
              dict(batch=2, ctx=1200, ctx_min=900), None),
}


@pytest.mark.parametrize("name", list(CASES))
def test_int4_append_and_decode_parity(name):
    base, over, max_splits = CASES[name]
    w = W.scaled(base, name="int4_" + name, **over) if over else base
    p = H.make_problem(w)
    _log(f"[int4] {name}: B={w.batch} Hq={w.num_q_heads} Hkv={w.num_kv_heads} lens={p.lens.tolist()}")
    cache, step = _run(p, max_splits)
    oc = _oracle_cache(p)
    pages = cache.pages.cpu().numpy()
    nd = int((pages != oc.pages).sum())
    assert nd == 0, f"{nd} INT4 page bytes differ"
    assert np.array_equal(cache.sinkwin.cpu().numpy().view(np.uint16), oc.sinkwin)
    ref, ref_lse = O.decode_attention(oc, p.table, np.arange(w.batch), p.lens, p.q, p.rot_k,
                                      p.rot_v, H.SM_SCALE)
    out, lse = step.out.cpu().numpy(), step.lse.cpu().numpy()
    rel = _row_err(out, ref)
    _log(f"[int4] {name}: max row rel err {rel.max():.3e}, max |dlse| {np.abs(lse - ref_lse).max():.3e}")
    assert np.all(np.isfinite(out))
    assert rel.max() <= TOL
    assert np.abs(lse - ref_lse).max() <= TOL


def test_int4_key_mean_append():
    w = W.scaled(W.WORKLOADS["qwen3_8b_b64"], name="int4_kmean", batch=2, ctx=700, ctx_min=400)
    p = H.make_problem(w)
    mu = W.key_channel_means(w)
    cache, step = _run(p, k_mean=mu)
    oc = _oracle_cache(p, mu)
    assert np.array_equal(cache.pages.cpu().numpy(), oc.pages)
    assert np.array_equal(cache.sinkwin.cpu().numpy().view(np.uint16), oc.sinkwin)


def test_int4_is_closer_to_exact_attention_than_int2():
    w = W.scaled(W.WORKLOADS["qwen3_4b"], name="int4_vs_int2", batch=2, ctx=1200, ctx_min=800)
    p = H.make_problem(w)
    _, s4 = _run(p)
    _, s2 = _run(p, bits=2)
    G = w.num_q_heads // w.num_kv_heads
    e4, e2 = [], []
    for b in range(w.batch):
        kb, vb = W.sequence_kv(w, b, int(p.lens[b]))
        for j in range(w.num_q_heads):
            o_ex, _, _ = O.softmax_attention(O.bf16_bits_to_f64(p.q[b, j]),
                                             O.bf16_bits_to_f64(kb[:, j // G]),
                                             O.bf16_bits_to_f64(vb[:, j // G]), H.SM_SCALE)
            scale = np.abs(o_ex).max()
            e4.append(np.abs(s4.out[b, j].cpu().numpy() - o_ex).max() / scale)
            e2.append(np.abs(s2.out[b, j].cpu().numpy() - o_ex).max() / scale)
    _log(f"[int4] error vs exact attention: INT4 {np.mean(e4):.4f}, INT2 {np.mean(e2):.4f}")
    assert np.mean(e4) < 0.5 * np.mean(e2)
