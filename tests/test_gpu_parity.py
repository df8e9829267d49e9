"""GPU parity: the HIP library against the CPU oracle on the same seeded inputs.

* Append: whole page pools and sink/window stores, pre-filled with a 0xA5 sentinel on both
  sides, must be equal byte for byte after the same appends (codes, fp16 scales/zeros, page
  placement, untouched bytes).
* Decode: out (fp32, rotated back) within 2e-3 normwise per (sequence, query head) row:
  max_c |gpu - oracle| / max_c |oracle|; lse within 2e-3.
Sizes span several pages and worker runs, ragged lengths and partial pages; worker counts go
from one worker for the whole batch (runs crossing many (sequence, head) pairs) to more
workers than pages; edge cases cover a context entirely in BF16, a single token, and a
partial-slot budget small enough to lengthen the runs.
"""
import dataclasses
import math
import sys

import numpy as np
import pytest
import torch

from oracle import oscar_oracle as O
from int2_rotated_kv_rotate_amd import harness as H
from int2_rotated_kv_rotate_amd import ops
from int2_rotated_kv_rotate_amd import workload as W

pytestmark = pytest.mark.gpu

TOL = 2e-3
SENTINEL = 0xA5
WS_FILL = 0xFF   # every float of a fresh workspace reads as NaN: nothing may depend on it


def _log(msg):
    print(msg, file=sys.stderr, flush=True)


def oracle_cache(p: H.Problem, k_mean=None, hadamard_signs=None):
    w = p.w
    cache = O.Cache(p.num_pages, w.num_kv_heads, w.batch, w.num_sink, w.window, fill=SENTINEL)
    needle = W.needle_site(w, p.lens)
    for b in range(w.batch):
        L = int(p.lens[b])
        kb, vb = W.sequence_kv(w, b, L, needle=needle, q_bits=p.q)
        rk, rv = (None, None) if hadamard_signs is not None else (p.rot_k, p.rot_v)
        cache.append(p.table[b], b, 0, kb[:L - 1], vb[:L - 1], rk, rv, w.clip, w.clip,
                     k_mean, hadamard_signs)
        cache.append(p.table[b], b, L - 1, kb[L - 1:], vb[L - 1:], rk, rv, w.clip,
                     w.clip, k_mean, hadamard_signs)
    return cache


def run_gpu(p: H.Problem, num_workers=0, max_splits=H.DEFAULT_MAX_SPLITS, k_mean=None,
            hadamard_signs=None):
    cache = H.GpuCache(p, fill=SENTINEL, k_mean=k_mean, hadamard_signs=hadamard_signs)
    last_k, last_v = cache.fill_context()
    step = H.DecodeStep(cache, num_workers=num_workers, max_splits=max_splits, ws_fill=WS_FILL)
    step.set_new_token(last_k, last_v)
    step.run()
    torch.cuda.synchronize()
    return cache, step


def row_errors(gpu, ref):
    err = np.abs(gpu.astype(np.float64) - ref).max(axis=-1)
    scale = np.abs(ref).max(axis=-1)
    return err / scale


def elem_errors(gpu, ref, floor=0.25):
    """Elementwise relative error with a floor: |gpu - ref| / max(|ref|, floor * max_row |ref|).
    For outputs of at least a quarter of their row's largest magnitude this is the plain
    relative error; below that (where relative error is unbounded near zero) it falls back to a
    quarter of the row scale."""
    ref = np.asarray(ref, np.float64)
    row = np.abs(ref).max(axis=-1, keepdims=True)
    return np.abs(gpu.astype(np.float64) - ref) / np.maximum(np.abs(ref), floor * row)


CASES = {
    # name: (workload, overrides, num_workers (0 = one per resident slot), max_splits)
    "tiny": (W.WORKLOADS["tiny"], {}, 0, 64),
    "q4b_ragged": (W.WORKLOADS["qwen3_4b"], dict(batch=2, ctx=1500, ctx_min=700), 7, 64),
    "q32b_g8": (W.WORKLOADS["qwen3_32b"], dict(batch=2, ctx=1000), 3, 64),
    "q32b_g8_ragged": (W.WORKLOADS["qwen3_32b"], dict(batch=5, ctx=900, ctx_min=100), 0, 64),
    # a key of 128 q/|q| mid-sequence: its logit (about 117 nats) exceeds the first page of its
    # run by more than the decode kernel's reference margin (and by more than fp32's range), so
    # that run is recomputed against its exact max; 3 workers keep the key away from the start
    # of a run
    "spike_recompute": (dataclasses.replace(W.WORKLOADS["qwen3_4b"], needle=True, needle_scale=128.0), dict(batch=2, ctx=1200, ctx_min=900), 3, 64),
    "spike_recompute_g8": (dataclasses.replace(W.WORKLOADS["qwen3_32b"], needle=True, needle_scale=128.0), dict(batch=2, ctx=1100, ctx_min=900), 3, 64),
    "q8b_more_workers_than_pages": (W.WORKLOADS["qwen3_8b_b64"], dict(batch=5, ctx=900, ctx_min=100), 5000, 64),
    "q8b_few_slots": (W.WORKLOADS["qwen3_8b_b64"], dict(batch=3, ctx=1200, ctx_min=600), 0, 3),
    "q8b_one_slot": (W.WORKLOADS["qwen3_8b_b64"], dict(batch=3, ctx=700, ctx_min=300), 0, 1),
    "all_bf16": (W.WORKLOADS["tiny"], dict(ctx=60), 0, 64),
    "one_token": (W.WORKLOADS["qwen3_4b"], dict(batch=1, ctx=1), 0, 64),
    "just_past_window": (W.WORKLOADS["qwen3_4b"], dict(batch=1, ctx=4 + 128 + 1), 1, 64),
    "page_multiple": (W.WORKLOADS["qwen3_4b"], dict(batch=2, ctx=16 * 20), 5, 64),
    "one_worker_many_pairs": (W.WORKLOADS["qwen3_8b_b64"], dict(batch=4, ctx=500, ctx_min=140), 1, 64),
    # other head groupings and sink/window geometries
    "g2": (dataclasses.replace(W.WORKLOADS["qwen3_4b"], num_q_heads=16), dict(batch=2, ctx=800, ctx_min=500), 0, 64),
    "g1_two_heads": (dataclasses.replace(W.WORKLOADS["tiny"], num_q_heads=2, num_kv_heads=2), dict(ctx=700), 0, 64),
    "no_sink_window16": (dataclasses.replace(W.WORKLOADS["qwen3_4b"], num_sink=0, window=16), dict(batch=2, ctx=900, ctx_min=600), 0, 64),
    "sink8_window1": (dataclasses.replace(W.WORKLOADS["qwen3_4b"], num_sink=8, window=1), dict(batch=2, ctx=640, ctx_min=400), 3, 64),
    # more sequences than one chunk of the work plan's prefix sums (256), short and ragged:
    # many have no INT2 page at all
    "batch_300_short": (dataclasses.replace(W.WORKLOADS["qwen3_4b"], num_q_heads=4, num_kv_heads=1), dict(batch=300, ctx=220, ctx_min=1), 0, 64),
}


@pytest.mark.parametrize("name", list(CASES))
def test_append_and_decode_parity(name):
    base, over, num_workers, max_splits = CASES[name]
    w = W.scaled(base, name=name, **over) if over else base
    p = H.make_problem(w)
    _log(f"[parity] {name}: B={w.batch} Hq={w.num_q_heads} Hkv={w.num_kv_heads} "
         f"lens={p.lens.tolist()} num_workers={num_workers} max_splits={max_splits}")
    cache, step = run_gpu(p, num_workers, max_splits)
    oc = oracle_cache(p)

    pages = cache.pages.cpu().numpy()
    mism = np.nonzero(pages != oc.pages)
    assert mism[0].size == 0, f"{mism[0].size} page bytes differ, first at {[m[:5] for m in mism]}"
    sw = cache.sinkwin.cpu().numpy().view(np.uint16)
    assert np.array_equal(sw, oc.sinkwin), "sink/window store differs"

    ref, ref_lse = O.decode_attention(oc, p.table, np.arange(w.batch), p.lens, p.q, p.rot_k,
                                      p.rot_v, H.SM_SCALE)
    out = step.out.cpu().numpy()
    lse = step.lse.cpu().numpy()
    rel = row_errors(out, ref)
    el = elem_errors(out, ref)
    _log(f"[parity] {name}: max row rel err {rel.max():.3e}, max elementwise {el.max():.3e}, "
         f"max |dlse| {np.abs(lse - ref_lse).max():.3e}")
    assert np.all(np.isfinite(out))
    assert rel.max() <= TOL
    assert el.max() <= TOL
    assert np.abs(lse - ref_lse).max() <= TOL


def test_key_mean_decode():
    """A cache whose keys had the workload's channel means removed before the rotation: pages
    equal to the oracle's, out within 2e-3 of the oracle's decode of that cache, lse of the
    centered logits; and the INT2 output is closer to the exact attention over the unquantised
    keys than without the mean (the point of removing it)."""
    w = W.scaled(W.WORKLOADS["qwen3_8b_b64"], name="kmean_decode", batch=3, ctx=1500, ctx_min=800)
    p = H.make_problem(w)
    mu = W.key_channel_means(w)
    cache, step = run_gpu(p, 0, H.DEFAULT_MAX_SPLITS, k_mean=mu)
    oc = oracle_cache(p, mu)
    assert np.array_equal(cache.pages.cpu().numpy(), oc.pages)
    assert np.array_equal(cache.sinkwin.cpu().numpy().view(np.uint16), oc.sinkwin)
    ref, ref_lse = O.decode_attention(oc, p.table, np.arange(w.batch), p.lens, p.q, p.rot_k,
                                      p.rot_v, H.SM_SCALE)
    out, lse = step.out.cpu().numpy(), step.lse.cpu().numpy()
    rel = row_errors(out, ref)
    _log(f"[parity] key mean: max row rel err {rel.max():.3e}, "
         f"max |dlse| {np.abs(lse - ref_lse).max():.3e}")
    assert rel.max() <= TOL
    assert elem_errors(out, ref).max() <= TOL
    assert np.abs(lse - ref_lse).max() <= TOL
    # against the exact attention over the unquantised, unrotated keys and values
    _, plain = run_gpu(p, 0, H.DEFAULT_MAX_SPLITS)
    err_c, err_p = [], []
    G = w.num_q_heads // w.num_kv_heads
    for b in range(w.batch):
        L = int(p.lens[b])
        kb, vb = W.sequence_kv(w, b, L)
        for j in range(w.num_q_heads):
            h = j // G
            q = O.bf16_bits_to_f64(p.q[b, j])
            o_ex, _, _ = O.softmax_attention(q, O.bf16_bits_to_f64(kb[:, h]),
                                             O.bf16_bits_to_f64(vb[:, h]), H.SM_SCALE)
            err_c.append(np.abs(out[b, j] - o_ex).max() / np.abs(o_ex).max())
            err_p.append(np.abs(plain.out.cpu().numpy()[b, j] - o_ex).max() / np.abs(o_ex).max())
    _log(f"[parity] key mean: error vs exact attention {np.mean(err_c):.4f} (centered) vs "
         f"{np.mean(err_p):.4f} (plain)")
    assert np.mean(err_c) < np.mean(err_p)


def test_hadamard_decode():
    """A cache written with the Hadamard-rotation append (fp64 fast transform, seeded signs),
    attended with its dense fp32 form as R_K and R_V: pages equal to the oracle's, outputs and
    lse within 2e-3 of the oracle's decode of that cache."""
    from int2_rotated_kv_rotate_amd import offline as OF
    w = W.scaled(W.WORKLOADS["qwen3_4b"], name="hadamard_decode", batch=2, ctx=1300, ctx_min=700)
    sk, sv = OF.hadamard_signs(70, w.num_kv_heads), OF.hadamard_signs(71, w.num_kv_heads)
    p = H.make_problem(w, rot_k=OF.hadamard_rotation(sk), rot_v=OF.hadamard_rotation(sv))
    cache, step = run_gpu(p, 0, H.DEFAULT_MAX_SPLITS, hadamard_signs=(sk, sv))
    oc = oracle_cache(p, hadamard_signs=(sk, sv))
    assert np.array_equal(cache.pages.cpu().numpy(), oc.pages)
    assert np.array_equal(cache.sinkwin.cpu().numpy().view(np.uint16), oc.sinkwin)
    ref, ref_lse = O.decode_attention(oc, p.table, np.arange(w.batch), p.lens, p.q, p.rot_k,
                                      p.rot_v, H.SM_SCALE)
    out, lse = step.out.cpu().numpy(), step.lse.cpu().numpy()
    rel = row_errors(out, ref)
    _log(f"[parity] hadamard: max row rel err {rel.max():.3e}, "
         f"max |dlse| {np.abs(lse - ref_lse).max():.3e}")
    assert rel.max() <= TOL
    assert elem_errors(out, ref).max() <= TOL
    assert np.abs(lse - ref_lse).max() <= TOL


def test_split_size_and_permutation_invariance():
    """Different worker counts agree to 1e-4; a permuted block table gives identical bits.

    Worker counts change where runs start (and with them the reference max and the fp32
    accumulation order), so results differ by rounding only.  The P.V accumulator carries the codes as 1 + code/4, a
    bias about 3.7x the signal that is removed after accumulation, and the normwise metric
    divides by max|o|, which is small for diffuse attention: ~1e-5 here, bounded by 1e-4."""
    w = W.scaled(W.WORKLOADS["qwen3_4b"], batch=2, ctx=1300, ctx_min=900, name="inv")
    p = H.make_problem(w)
    _, s1 = run_gpu(p, 4)
    _, s2 = run_gpu(p, 33)
    _, s0 = run_gpu(p, 0)
    assert row_errors(s0.out.cpu().numpy(), s2.out.cpu().numpy().astype(np.float64)).max() <= 1e-4
    a, b = s1.out.cpu().numpy(), s2.out.cpu().numpy()
    assert row_errors(a, b.astype(np.float64)).max() <= 1e-4
    # same physical content, different page ids
    rng = np.random.default_rng(5)
    perm = rng.permutation(p.num_pages).astype(np.int32)
    p2 = H.Problem(p.w, p.lens, np.where(p.table >= 0, perm[np.maximum(p.table, 0)], -1).astype(np.int32),
                   p.num_pages, p.rot_k, p.rot_v, p.q)
    _, s3 = run_gpu(p2, 4)
    assert np.array_equal(a, s3.out.cpu().numpy())
    # run-to-run determinism
    s1.attend()
    torch.cuda.synchronize()
    assert np.array_equal(a, s1.out.cpu().numpy())


def test_distinct_k_and_v_rotations_are_not_conflated():
    w = W.scaled(W.WORKLOADS["qwen3_4b"], batch=1, ctx=400, name="kv_rot")
    p = H.make_problem(w)
    assert not np.allclose(p.rot_k, p.rot_v)
    _, step = run_gpu(p, 8)
    oc = oracle_cache(p)
    ref, _ = O.decode_attention(oc, p.table, [0], p.lens, p.q, p.rot_k, p.rot_v, H.SM_SCALE)
    assert row_errors(step.out.cpu().numpy(), ref).max() <= TOL
    # and using R_K for the output rotation would be far off
    wrong, _ = O.decode_attention(oc, p.table, [0], p.lens, p.q, p.rot_k, p.rot_k, H.SM_SCALE)
    assert row_errors(step.out.cpu().numpy(), wrong).max() > 0.1


def _combine_and_check(B, hq, hkv, max_splits, valid, nvalid, seed):
    """Seeded partials in a fresh workspace (stale INT2 slots past each pair's nvalid hold NaN
    outputs, a large m and an l of 7 or NaN), oscar_combine, and the oracle merge of the slots
    each (sequence, query head) uses, rotated by R_V^T."""
    nslots = max_splits + ops.WINDOW_SLOTS
    G = hq // hkv
    m, l, o = W.synthetic_partials(seed, B, hq, nslots, valid)
    for b in range(B):
        for j in range(hq):
            stale = np.arange(nvalid[b, j // G], max_splits)
            o[b, j, stale] = np.nan
            m[b, j, stale] = 1e30
            l[b, j, stale] = 7.0 if j % 2 == 0 else np.nan
    rot_v = W.rotations(W.scaled(W.WORKLOADS["qwen3_4b"], name="rv"), "v")[:hkv].astype(np.float32)
    nbytes = ops.decode_workspace_bytes(B, hq, max_splits)
    ws = np.zeros(nbytes, np.uint8)
    qb = B * hq * 1024
    ob = B * hq * nslots * 128 * 4
    ws[qb:qb + ob] = o.astype(np.float32).reshape(-1).view(np.uint8)
    ml = np.stack([m, l], axis=-1).astype(np.float32)
    ws[qb + ob:qb + ob + ml.nbytes] = ml.reshape(-1).view(np.uint8)
    # plan region: 4 header words, pstart/npg/pglo [B] each, then nvalid [B][hkv]
    nv_off = qb + ob + ml.nbytes + 4 * (4 + 3 * B)
    ws[nv_off:nv_off + nvalid.nbytes] = nvalid.astype(np.int32).reshape(-1).view(np.uint8)
    dws = torch.from_numpy(ws).cuda()
    out = torch.empty((B, hq, 128), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, hq), dtype=torch.float32, device="cuda")
    ops.combine(B, hq, hkv, max_splits, dws, torch.from_numpy(rot_v).cuda(), out, lse)
    torch.cuda.synchronize()
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    for b in range(B):
        for j in range(hq):
            used = list(range(nvalid[b, j // G])) + list(range(max_splits, nslots))
            if not valid[b, used].any():
                assert np.all(out[b, j] == 0) and lse[b, j] == -np.inf
                continue
            o_ref, lse_ref = O.merge_partials(m[b, j, used], l[b, j, used], o[b, j, used])
            o_ref = o_ref @ rot_v[j // G].astype(np.float64).T
            assert np.abs(out[b, j] - o_ref).max() <= 1e-5 * max(1, np.abs(o_ref).max()), (b, j)
            assert abs(lse[b, j] - lse_ref) <= 1e-5 * max(1, abs(lse_ref)), (b, j)


@pytest.mark.parametrize("max_splits,nvalid_rows", [
    (5, [[5, 3], [2, 0], [4, 5]]),            # one workgroup per KV head
    (100, [[100, 37], [2, 0], [99, 64]]),     # few pairs, many splits: one per query head
])
def test_combine_with_synthetic_partials(max_splits, nvalid_rows):
    """oscar_combine on seeded partials (not produced by the library) vs the oracle merge.

    Each (sequence, KV head) pair declares how many INT2 slots it filled (the plan's nvalid);
    slots past that hold NaN outputs, a large m and an l of 7 or NaN, and must not be read.
    The window slots that follow are all merged, some of them empty."""
    B, hq, hkv = 3, 8, 2
    nslots = max_splits + ops.WINDOW_SLOTS
    valid = np.ones((B, nslots), bool)
    valid[0, 2] = False
    valid[0, 3:max_splits:7] = False
    valid[0, max_splits + 1] = False         # an empty window part between two full ones
    valid[0, max_splits + 5:] = False        # window parts the launch did not use
    valid[1, 1:] = False
    valid[2, :] = False                      # a row with no positions at all
    _combine_and_check(B, hq, hkv, max_splits, valid, np.array(nvalid_rows, np.int32), 42)


# (batch, query heads, KV heads, max_splits): the per-KV-head form for every group size with a
# last workgroup of fewer than 8 / G sequences, with more slots than its lanes hold (past 128),
# and the per-query-head form with more slots than its 1024 threads (past 1024).
COMBINE_FORMS = {
    "kv_g1": (3, 2, 2, 20),
    "kv_g2": (5, 4, 2, 20),
    "kv_g8": (3, 16, 2, 20),
    "kv_g4_200_slots": (16, 32, 8, 200),
    "head_g1_1100_slots": (1, 2, 2, 1100),
}


@pytest.mark.parametrize("name", list(COMBINE_FORMS))
def test_combine_forms(name):
    """oscar_combine against the oracle merge in each of its launch forms and slot-count
    regimes: seeded nvalid per (sequence, KV head) (including 0 and max_splits), ~10% of the
    used slots empty, a random subset of the window slots used."""
    B, hq, hkv, max_splits = COMBINE_FORMS[name]
    rng = np.random.default_rng(7)
    nslots = max_splits + ops.WINDOW_SLOTS
    valid = rng.random((B, nslots)) > 0.1
    nvalid = rng.integers(0, max_splits + 1, (B, hkv)).astype(np.int32)
    nvalid.reshape(-1)[0] = max_splits
    if nvalid.size > 1:
        nvalid.reshape(-1)[1] = 0
    _combine_and_check(B, hq, hkv, max_splits, valid, nvalid, 43)


@pytest.mark.parametrize("name,over,split_pages",
                         [("bf16_q4b", dict(batch=2, ctx=1100, ctx_min=500), 8),
                          ("bf16_q32b", dict(batch=2, ctx=700), 16)])
def test_bf16_baseline_parity(name, over, split_pages):
    base = W.WORKLOADS["qwen3_32b" if "q32b" in name else "qwen3_4b"]
    w = W.scaled(base, name=name, **over)
    p = H.make_problem(w)
    _log(f"[parity] {name}: lens={p.lens.tolist()}")
    hkv = w.num_kv_heads
    lay = ops.make_layout(hkv, 0, 0, p.num_pages, p.table.shape[1], w.batch)
    pages = torch.full((p.num_pages, hkv, O.BF16_PAGE_ELEMS), 0x5A5A, dtype=torch.int16, device="cuda")
    opages = np.full((p.num_pages, hkv, O.BF16_PAGE_ELEMS), 0x5A5A, np.uint16)
    ks, vs = [], []
    for b in range(w.batch):
        kb, vb = W.sequence_kv(w, b, int(p.lens[b]))
        ks.append(kb)
        vs.append(vb)
        for pos in range(int(p.lens[b])):
            for h in range(hkv):
                O.bf16_write_token(opages[p.table[b, pos // 16], h], pos % 16, kb[pos, h], vb[pos, h])
    offs = np.zeros(w.batch + 1, np.int32)
    offs[1:] = np.cumsum(p.lens)
    table = torch.from_numpy(p.table).cuda()
    ops.bf16_append(lay, pages, table, H.as_i16(np.concatenate(ks)).cuda(),
                    H.as_i16(np.concatenate(vs)).cuda(), torch.from_numpy(offs).cuda(),
                    torch.zeros(w.batch, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert np.array_equal(pages.cpu().numpy().view(np.uint16), opages)
    max_splits = int(math.ceil(p.table.shape[1] / split_pages))
    ws = torch.full((ops.decode_workspace_bytes(w.batch, w.num_q_heads, max_splits),), WS_FILL,
                    dtype=torch.uint8, device="cuda")
    q = H.as_i16(p.q).cuda()
    lens = torch.from_numpy(p.lens.astype(np.int32)).cuda()
    ops.bf16_decode_attention(lay, pages, table, q, lens, H.SM_SCALE, split_pages, max_splits, ws)
    out = torch.empty((w.batch, w.num_q_heads, 128), dtype=torch.float32, device="cuda")
    lse = torch.empty((w.batch, w.num_q_heads), dtype=torch.float32, device="cuda")
    ops.combine(w.batch, w.num_q_heads, hkv, max_splits, ws, None, out, lse)
    torch.cuda.synchronize()
    ref, ref_lse = O.bf16_decode_attention(opages, p.table, p.lens, p.q, H.SM_SCALE, hkv)
    rel = row_errors(out.cpu().numpy(), ref)
    _log(f"[parity] {name}: max row rel err {rel.max():.3e}")
    assert rel.max() <= TOL
    assert elem_errors(out.cpu().numpy(), ref).max() <= TOL
    assert np.abs(lse.cpu().numpy() - ref_lse).max() <= TOL
