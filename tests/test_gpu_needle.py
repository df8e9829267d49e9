"""Planted-needle check at 128K context (batch 1, 32 query / 8 KV heads, sink 4 + window 128).

One seeded key row in the middle of the context (position L/2, a seeded KV head h* and query
head j* of its group) is set to bf16(8 q_j* / |q_j*|) before it is appended.  Its attention
weight is w = exp(z - lse), where z is the needle's logit from its stored codes (the oracle's,
which the GPU's page records must equal byte for byte) and lse is the log-sum-exp of all the
head's logits: the GPU's lse (from oscar_combine) must give the oracle's weight to 2e-3
relative.  (Among 131K positions with ×15 outlier key channels the needle's weight is small,
about 1e-5 here; the check is the agreement, not its size.)  The output rows of the needle's
KV head must also match the oracle to 2e-3.

A second reading of "its attention weight" goes through the value path: the needle position is
appended again with the same key and two different value rows (large, so that the needle's
share of the output stands well above rounding), the sink/window store is restored after each
re-append (the re-append makes the position the newest and writes a window row), and the
decode is run for each.  Keys are unchanged, so the weights are; the output difference is then
w * (v2 - v1) . R_V^T for the dequantised rotated rows v1, v2 the oracle stores, and
w = <out2 - out1, (v2 - v1) R_V^T> / |v2 - v1|^2 must equal the oracle's weight to 2e-3
relative.
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


@pytest.fixture(scope="module")
def needle_run():
    w = W.WORKLOADS["long_128k"]
    p = H.make_problem(w)
    cache = H.GpuCache(p, fill=SENTINEL)
    last_k, last_v = cache.fill_context()
    step = H.DecodeStep(cache, ws_fill=0xFF)
    step.set_new_token(last_k, last_v)
    step.run()
    torch.cuda.synchronize()
    return w, p, cache, step


def test_needle_weight_128k(needle_run):
    w, p, cache, step = needle_run
    b, pos, h, j = W.needle_site(w, p.lens)
    L = int(p.lens[b])
    G = w.group
    _log(f"[needle] L={L} position {pos} KV head {h} query head {j}")

    kb, vb = W.sequence_kv(w, b, L, offsets=W.key_offsets(w), outliers=W.outlier_channels(w),
                           needle=(b, pos, h, j), q_bits=p.q)
    oc = O.Cache(p.num_pages, 1, w.batch, w.num_sink, w.window, fill=SENTINEL)
    args = (p.rot_k[h:h + 1], p.rot_v[h:h + 1], w.clip, w.clip)
    oc.append(p.table[b], b, 0, kb[:L - 1, h:h + 1], vb[:L - 1, h:h + 1], *args)
    oc.append(p.table[b], b, L - 1, kb[L - 1:, h:h + 1], vb[L - 1:, h:h + 1], *args)

    pages_b = p.table[b, :math.ceil(L / 16)]
    idx = torch.from_numpy(pages_b.astype(np.int64)).to(cache.pages.device)
    assert np.array_equal(cache.pages[idx, h].cpu().numpy(), oc.pages[pages_b, 0])

    ref, ref_lse = O.decode_attention(oc, p.table[b:b + 1], np.array([b]), p.lens[b:b + 1],
                                      p.q[b:b + 1, h * G:(h + 1) * G], p.rot_k[h:h + 1],
                                      p.rot_v[h:h + 1], H.SM_SCALE)
    # the needle's logit from its stored (dequantised) key in the rotated frame
    k_all, _, _ = oc.read_sequence(p.table[b], b, 0, L)
    qr = O.rotate_query(p.q[b], p.rot_k, G)[j]
    z = H.SM_SCALE * float(k_all[pos] @ qr)
    lse_gpu = float(step.lse[b, j].item())
    lse_ref = float(ref_lse[0, j - h * G])
    w_ref = math.exp(z - lse_ref)
    w_gpu = math.exp(z - lse_gpu)
    _log(f"[needle] logit {z:.4f}, lse oracle {lse_ref:.4f} gpu {lse_gpu:.4f}; weight oracle "
         f"{w_ref:.4e} gpu {w_gpu:.4e} (rel {abs(w_gpu / w_ref - 1):.2e})")
    assert w_ref > 0.0
    assert abs(w_gpu / w_ref - 1.0) <= TOL

    out = step.out[b, h * G:(h + 1) * G].cpu().numpy().astype(np.float64)
    rel = np.abs(out - ref[0]).max(axis=-1) / np.abs(ref[0]).max(axis=-1)
    _log(f"[needle] KV head {h}: max row rel err {rel.max():.3e}")
    assert rel.max() <= TOL


def test_needle_weight_by_value_swap(needle_run):
    w, p, cache, step = needle_run
    b, pos, h, j = W.needle_site(w, p.lens)
    L = int(p.lens[b])
    G = w.group
    kb, vb = W.sequence_kv(w, b, L, offsets=W.key_offsets(w), outliers=W.outlier_channels(w),
                           needle=(b, pos, h, j), q_bits=p.q)
    # the oracle's weight of the needle (as in the test above)
    oc = O.Cache(p.num_pages, 1, w.batch, w.num_sink, w.window, fill=SENTINEL)
    args = (p.rot_k[h:h + 1], p.rot_v[h:h + 1], w.clip, w.clip)
    oc.append(p.table[b], b, 0, kb[:L - 1, h:h + 1], vb[:L - 1, h:h + 1], *args)
    oc.append(p.table[b], b, L - 1, kb[L - 1:, h:h + 1], vb[L - 1:, h:h + 1], *args)
    _, ref_lse = O.decode_attention(oc, p.table[b:b + 1], np.array([b]), p.lens[b:b + 1],
                                    p.q[b:b + 1, h * G:(h + 1) * G], p.rot_k[h:h + 1],
                                    p.rot_v[h:h + 1], H.SM_SCALE)
    k_all, _ = oc.read_sequence(p.table[b], b, 0, L)[:2]
    qr = O.rotate_query(p.q[b], p.rot_k, G)[j]
    w_ref = math.exp(H.SM_SCALE * float(k_all[pos] @ qr) - float(ref_lse[0, j - h * G]))

    # two value rows for the needle position (seeded, about 1000 in magnitude), same key
    rng = np.random.default_rng(77)
    snap = cache.sinkwin.clone()
    outs, vhat = [], []
    for t in range(2):
        k_rows = kb[pos:pos + 1].copy()
        v_rows = vb[pos:pos + 1].copy()
        v_rows[0, h] = O.f32_to_bf16_bits((rng.standard_normal(128) * 1000.0).astype(np.float32))
        cache.append([k_rows], [v_rows], [pos])
        cache.sinkwin.copy_(snap)          # undo the window row the re-append wrote
        step.attend()
        torch.cuda.synchronize()
        outs.append(step.out[b, j].cpu().numpy().astype(np.float64))
        oc.append(p.table[b], b, pos, k_rows[:, h:h + 1], v_rows[:, h:h + 1], *args)
        vhat.append(oc.read_sequence(p.table[b], b, 0, L)[1][pos])   # pos is an INT2 position
        # the GPU's record of the needle's page equals the oracle's after the re-append
        pg = int(p.table[b, pos // 16])
        assert np.array_equal(cache.pages[pg, h].cpu().numpy(), oc.pages[pg, 0])
    dv = (vhat[1] - vhat[0]) @ p.rot_v[h].astype(np.float64).T
    w_swap = float((outs[1] - outs[0]) @ dv / (dv @ dv))
    _log(f"[needle] value swap: |dv| {np.linalg.norm(dv):.1f}, weight oracle {w_ref:.4e} gpu "
         f"{w_swap:.4e} (rel {abs(w_swap / w_ref - 1):.2e})")
    assert abs(w_swap / w_ref - 1.0) <= TOL
