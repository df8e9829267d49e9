"""The append kernels write the same bytes: fp64 on the vector ALUs, and the matrix cores with a
bounded error and exact recomputation of whatever the bound cannot certify.

Every case appends the same rows with OSCAR_APPEND_VECTOR and OSCAR_APPEND_MATRIX into pools
pre-filled with a 0xA5 sentinel; the page pools and sink/window stores must be equal byte for
byte, and (except at the full prefill size) equal to the oracle's.

Cases:
  * the Qwen3-8B layer workload (per-channel offsets, x15 outlier key channels), ragged
    lengths, one call per batch;
  * special rotations: identity and a signed permutation (rotation exact in any order), an
    orthogonal matrix scaled by 2.5 (column norms far from 1), and the offline spectral
    rotation (eigenbasis of a calibration covariance) with the calibrated key mean;
  * special rows with a seeded orthogonal rotation: rows along a column of R (every other
    rotated value is tiny next to ||x||, so scales, zeros, codes and BF16 copies are uncertain
    and recomputed), zero rows, subnormal rows, a huge dynamic range within a row;
  * groups with max == -min (a code threshold exactly at zero), one-signed and constant groups;
  * keys with a mean removed before the rotation (workload means, a large random mean, zero,
    and the special rows with a mean);
  * the Hadamard-rotation append (its own kernel) against the oracle;
  * the full prefill shape: 64 sequences x 2048 new tokens at the end of 16K-32K contexts,
    the two kernels against each other over all 2.1 million rows, and sampled (sequence, KV
    head) pairs against the oracle (their rows copied to the host).
"""
import sys

import numpy as np
import pytest
import torch

from oracle import oscar_oracle as O
from int2_rotated_kv_rotate_amd import harness as H
from int2_rotated_kv_rotate_amd import offline as OF
from int2_rotated_kv_rotate_amd import ops
from int2_rotated_kv_rotate_amd import workload as W

pytestmark = pytest.mark.gpu

SENTINEL = 0xA5


def _log(msg):
    print(msg, file=sys.stderr, flush=True)


def _append_both(p, k_rows, v_rows, start, k_mean=None):
    """GPU caches after appending with each method (one call each)."""
    out = {}
    for method in (ops.APPEND_VECTOR, ops.APPEND_MATRIX):
        c = H.GpuCache(p, fill=SENTINEL, k_mean=k_mean)
        c.append(k_rows, v_rows, start, method=method)
        torch.cuda.synchronize()
        out[method] = (c.pages.cpu().numpy(), c.sinkwin.cpu().numpy().view(np.uint16))
    return out


def _oracle(p, k_rows, v_rows, start, k_mean=None):
    w = p.w
    oc = O.Cache(p.num_pages, w.num_kv_heads, w.batch, w.num_sink, w.window, fill=SENTINEL)
    for b in range(w.batch):
        if k_rows[b].shape[0]:
            oc.append(p.table[b], b, int(start[b]), k_rows[b], v_rows[b], p.rot_k, p.rot_v,
                      w.clip, w.clip, k_mean)
    return oc


def _check(name, p, k_rows, v_rows, start, with_oracle=True, k_mean=None):
    res = _append_both(p, k_rows, v_rows, start, k_mean)
    (pv, sv), (pm, sm) = res[ops.APPEND_VECTOR], res[ops.APPEND_MATRIX]
    nd = int((pv != pm).sum())
    _log(f"[append] {name}: {sum(r.shape[0] for r in k_rows)} rows; vector vs matrix: "
         f"{nd} page bytes differ, sink/window equal: {np.array_equal(sv, sm)}")
    assert nd == 0
    assert np.array_equal(sv, sm)
    if with_oracle:
        oc = _oracle(p, k_rows, v_rows, start, k_mean)
        assert np.array_equal(pm, oc.pages), f"{int((pm != oc.pages).sum())} bytes differ from the oracle"
        assert np.array_equal(sm, oc.sinkwin)


def _workload_rows(w, lens):
    offsets, outliers = W.key_offsets(w), W.outlier_channels(w)
    ks, vs = [], []
    for b in range(w.batch):
        kb, vb = W.sequence_kv(w, b, int(lens[b]), offsets=offsets, outliers=outliers)
        ks.append(kb)
        vs.append(vb)
    return ks, vs


def test_workload_rows():
    w = W.scaled(W.WORKLOADS["qwen3_8b_b64"], name="append_methods", batch=3, ctx=1500, ctx_min=700)
    p = H.make_problem(w)
    ks, vs = _workload_rows(w, p.lens)
    _check("workload", p, ks, vs, [0] * w.batch)


def _signed_permutation(rng, hkv):
    out = np.zeros((hkv, 128, 128), dtype=np.float64)
    for h in range(hkv):
        perm = rng.permutation(128)
        out[h, np.arange(128), perm] = rng.choice([-1.0, 1.0], size=128)
    return out


@pytest.mark.parametrize("kind", ["identity", "signed_permutation", "scaled", "spectral"])
def test_special_rotations(kind):
    w = W.scaled(W.WORKLOADS["qwen3_4b"], name="append_rot_" + kind, batch=2, ctx=700, ctx_min=300)
    rng = np.random.default_rng(11)
    k_mean = None
    if kind == "spectral":   # offline calibration on another sequence's rows, keys centered
        wc = W.scaled(W.WORKLOADS["qwen3_4b"], name="calib", batch=3, ctx=1024)
        kc, vc = W.sequence_kv(wc, 2, 1024)
        rk, rv, k_mean = OF.calibrate(kc, vc)
    elif kind == "identity":
        rk = np.broadcast_to(np.eye(128), (w.num_kv_heads, 128, 128)).copy()
        rv = rk.copy()
    elif kind == "signed_permutation":
        rk, rv = _signed_permutation(rng, w.num_kv_heads), _signed_permutation(rng, w.num_kv_heads)
    else:
        rk, rv = 2.5 * W.rotations(w, "k"), 2.5 * W.rotations(w, "v")
    p = H.make_problem(w, rot_k=rk, rot_v=rv)
    ks, vs = _workload_rows(w, p.lens)
    _check(kind, p, ks, vs, [0] * w.batch, k_mean=k_mean)


def _special_rows(rng, rot32, n):
    """[n][Hkv][128] bf16 bits: rows along a column of R (scaled), zeros, subnormals, and rows
    mixing 2^-20 and 2^8 magnitudes, in a seeded order."""
    hkv = rot32.shape[0]
    x = np.empty((n, hkv, 128), dtype=np.float32)
    kinds = rng.integers(0, 4, size=n)
    for i in range(n):
        for h in range(hkv):
            k = kinds[i]
            if k == 0:      # x = a * R[:, j]^T: rotated value a at channel j, ~0 elsewhere
                j = rng.integers(0, 128)
                x[i, h] = rot32[h, :, j] * np.float32(rng.uniform(0.5, 20.0))
            elif k == 1:
                x[i, h] = 0.0
            elif k == 2:    # bf16 subnormals (fp32 subnormal range)
                x[i, h] = rng.standard_normal(128).astype(np.float32) * np.float32(2.0 ** -130)
            else:
                big = rng.random(128) < 0.1
                x[i, h] = np.where(big, 256.0, 2.0 ** -20) * rng.standard_normal(128)
    return W.to_bf16_bits(x)


def test_special_rows():
    w = W.scaled(W.WORKLOADS["qwen3_4b"], name="append_special_rows", batch=2, ctx=600, ctx_min=500)
    p = H.make_problem(w)
    rng = np.random.default_rng(12)
    ks = [_special_rows(rng, p.rot_k, int(L)) for L in p.lens]
    vs = [_special_rows(rng, p.rot_v, int(L)) for L in p.lens]
    _check("special_rows", p, ks, vs, [0] * w.batch)


@pytest.mark.parametrize("kind", ["workload_means", "large_random", "zero"])
def test_key_mean(kind):
    """Keys with a mean removed before the rotation: the workload's channel means, a large
    random mean (|mu| ~ 30, so the centered values are small next to both terms), and a zero
    mean (which must give exactly the bytes of no mean)."""
    w = W.scaled(W.WORKLOADS["qwen3_8b_b64"], name="append_kmean", batch=2, ctx=900, ctx_min=500)
    p = H.make_problem(w)
    ks, vs = _workload_rows(w, p.lens)
    if kind == "workload_means":
        mu = W.key_channel_means(w)
    elif kind == "large_random":
        mu = (np.random.default_rng(21).standard_normal((w.num_kv_heads, 128)) * 30).astype(np.float32)
    else:
        mu = np.zeros((w.num_kv_heads, 128), np.float32)
    _check("key_mean_" + kind, p, ks, vs, [0] * w.batch, k_mean=mu)
    if kind == "zero":
        plain = _oracle(p, ks, vs, [0] * w.batch)
        centered = _oracle(p, ks, vs, [0] * w.batch, mu)
        assert np.array_equal(plain.pages, centered.pages)


def test_key_mean_special_rows():
    """The special rows (see _special_rows) with a seeded mean: the certification of scales,
    zeros, codes and BF16 copies with the mean's rounding in the error bound."""
    w = W.scaled(W.WORKLOADS["qwen3_4b"], name="append_kmean_special", batch=2, ctx=600, ctx_min=500)
    p = H.make_problem(w)
    rng = np.random.default_rng(22)
    ks = [_special_rows(rng, p.rot_k, int(L)) for L in p.lens]
    vs = [_special_rows(rng, p.rot_v, int(L)) for L in p.lens]
    mu = (rng.standard_normal((w.num_kv_heads, 128)) * 3).astype(np.float32)
    mu[0, :64] = 0.0                     # some channels without a mean
    _check("key_mean_special_rows", p, ks, vs, [0] * w.batch, k_mean=mu)


def _dense_hadamard(signs, hkv):
    """[Hkv][128][128] dense form (what attention reads) of the Hadamard rotation."""
    if signs is None:
        return np.broadcast_to(OF.hadamard_rotation(None), (hkv, 128, 128)).copy()
    return OF.hadamard_rotation(signs)


@pytest.mark.parametrize("kind", ["workload", "special_rows", "no_signs"])
def test_hadamard_append(kind):
    """The Hadamard-rotation append (fp64 fast transform) against the oracle, byte for byte:
    workload rows with seeded signs, the special rows (zero, subnormal, high dynamic range), and
    all signs +1.  Whole contexts, so every call writes sink, window and bulk rows."""
    w = W.scaled(W.WORKLOADS["qwen3_8b_b64"], name="append_hadamard_" + kind, batch=3, ctx=1100,
                 ctx_min=300)
    sk, sv = (None, None) if kind == "no_signs" else (OF.hadamard_signs(60, w.num_kv_heads),
                                                      OF.hadamard_signs(61, w.num_kv_heads))
    p = H.make_problem(w, rot_k=_dense_hadamard(sk, w.num_kv_heads),
                       rot_v=_dense_hadamard(sv, w.num_kv_heads))
    if kind == "special_rows":
        rng = np.random.default_rng(62)
        ks = [_special_rows(rng, p.rot_k, int(L)) for L in p.lens]
        vs = [_special_rows(rng, p.rot_v, int(L)) for L in p.lens]
    else:
        ks, vs = _workload_rows(w, p.lens)
    c = H.GpuCache(p, fill=SENTINEL, hadamard_signs=(sk, sv))
    c.append(ks, vs, [0] * w.batch)
    torch.cuda.synchronize()
    oc = O.Cache(p.num_pages, w.num_kv_heads, w.batch, w.num_sink, w.window, fill=SENTINEL)
    for b in range(w.batch):
        oc.append(p.table[b], b, 0, ks[b], vs[b], None, None, w.clip, w.clip,
                  hadamard_signs=(sk, sv))
    pages = c.pages.cpu().numpy()
    nd = int((pages != oc.pages).sum())
    _log(f"[append] hadamard {kind}: {sum(k.shape[0] for k in ks)} rows, {nd} page bytes differ")
    assert nd == 0
    assert np.array_equal(c.sinkwin.cpu().numpy().view(np.uint16), oc.sinkwin)


def test_symmetric_groups():
    """Identity rotation, rows whose every 32-channel group has max == -min (so a code threshold
    sits exactly at zero, where fp32 values are densest), plus rows whose groups are one-signed
    or constant."""
    w = W.scaled(W.WORKLOADS["qwen3_4b"], name="append_symmetric", batch=2, ctx=520, ctx_min=400)
    eye = np.broadcast_to(np.eye(128), (w.num_kv_heads, 128, 128)).copy()
    p = H.make_problem(w, rot_k=eye, rot_v=eye)
    rng = np.random.default_rng(13)

    def rows(n):
        x = rng.uniform(-1.0, 1.0, size=(n, w.num_kv_heads, 4, 32)).astype(np.float32)
        a = np.float32(2.0) ** rng.integers(-8, 8, size=(n, w.num_kv_heads, 4, 1)).astype(np.float32)
        x *= a
        kind = rng.integers(0, 4, size=(n, w.num_kv_heads, 4))
        x[..., 0] = np.where(kind < 2, a[..., 0], x[..., 0])      # max = a, min = -a
        x[..., 1] = np.where(kind < 2, -a[..., 0], x[..., 1])
        x = np.where((kind == 2)[..., None], np.abs(x), x)        # one-signed group
        x = np.where((kind == 3)[..., None], a, x)                # constant group
        return W.to_bf16_bits(x.reshape(n, w.num_kv_heads, 128))

    ks = [rows(int(L)) for L in p.lens]
    vs = [rows(int(L)) for L in p.lens]
    _check("symmetric_groups", p, ks, vs, [0] * w.batch)


def test_chunked_appends_with_window_rows():
    """Appends of 300 rows after existing contexts: every call has sink, window and bulk rows
    on both methods; the oracle applies the same calls."""
    w = W.scaled(W.WORKLOADS["qwen3_8b_b64"], name="append_chunks", batch=2, ctx=1400, ctx_min=1000)
    p = H.make_problem(w)
    ks, vs = _workload_rows(w, p.lens)
    caches = {m: H.GpuCache(p, fill=SENTINEL) for m in (ops.APPEND_VECTOR, ops.APPEND_MATRIX)}
    oc = O.Cache(p.num_pages, w.num_kv_heads, w.batch, w.num_sink, w.window, fill=SENTINEL)
    pos = [0] * w.batch
    while any(pos[b] < p.lens[b] for b in range(w.batch)):
        kc, vc, st = [], [], []
        for b in range(w.batch):
            e = min(int(p.lens[b]), pos[b] + 300)
            kc.append(ks[b][pos[b]:e])
            vc.append(vs[b][pos[b]:e])
            st.append(pos[b])
            if e > pos[b]:
                oc.append(p.table[b], b, pos[b], ks[b][pos[b]:e], vs[b][pos[b]:e], p.rot_k,
                          p.rot_v, w.clip, w.clip)
            pos[b] = e
        for m, c in caches.items():
            c.append(kc, vc, st, method=m)
    torch.cuda.synchronize()
    for m, c in caches.items():
        assert np.array_equal(c.pages.cpu().numpy(), oc.pages), f"method {m}"
        assert np.array_equal(c.sinkwin.cpu().numpy().view(np.uint16), oc.sinkwin), f"method {m}"


def _full_prefill_inputs():
    """The benchmark's prefill: 64 sequences x 2048 new tokens at positions [L - 2048, L), L in
    [16384, 32768].  Rows follow the workload recipe (N(0,1) + per-channel N(0,2) key offsets,
    x15 outlier key channels), drawn on the GPU from a seeded generator."""
    w = W.WORKLOADS["qwen3_8b_b64"]
    p = H.make_problem(w)
    n_new = w.prefill_new
    gen = torch.Generator(device="cuda")
    gen.manual_seed(2048)
    hkv = w.num_kv_heads
    total = n_new * w.batch
    k = torch.randn((total, hkv, 128), generator=gen, device="cuda")
    k += torch.from_numpy(W.key_offsets(w)).cuda()[None]
    out_ch = torch.from_numpy(W.outlier_channels(w)).cuda()
    for h in range(hkv):
        k[:, h, out_ch[h]] *= 15.0
    v = torch.randn((total, hkv, 128), generator=gen, device="cuda")
    k16 = k.to(torch.bfloat16).view(torch.int16).contiguous()
    v16 = v.to(torch.bfloat16).view(torch.int16).contiguous()
    offs = torch.arange(0, total + 1, n_new, dtype=torch.int32, device="cuda")
    start = torch.from_numpy((p.lens - n_new).astype(np.int32)).cuda()
    return w, p, n_new, total, k16, v16, offs, start


def test_full_prefill_shape():
    """The full prefill the benchmark times (see _full_prefill_inputs): both append methods byte
    for byte, and sampled (sequence, KV head) pairs against the oracle."""
    w, p, n_new, total, k16, v16, offs, start = _full_prefill_inputs()
    res = {}
    for m in (ops.APPEND_VECTOR, ops.APPEND_MATRIX):
        c = H.GpuCache(p, fill=SENTINEL)
        ops.rotate_quantize_append(c.layout, c.pages, c.sinkwin, c.table, c.slots, k16, v16, offs,
                                   start, c.rot_k, c.rot_v, w.clip, w.clip, method=m)
        torch.cuda.synchronize()
        res[m] = (c.pages, c.sinkwin)
    (pv, sv), (pm, sm) = res[ops.APPEND_VECTOR], res[ops.APPEND_MATRIX]
    nd = int((pv != pm).sum().item())
    _log(f"[append] full prefill {total} rows: {nd} page bytes differ")
    assert nd == 0
    assert torch.equal(sv, sm)
    # the appended pages really were written (sentinel replaced in the tail's records)
    b = 0
    last_page = int(p.table[b, (int(p.lens[b]) - 1) // 16])
    assert not bool((pm[last_page, 0, :1024] == SENTINEL).all().item())
    # sampled (sequence, KV head) pairs against the oracle: the pair's 2048 rows appended at
    # the same positions into a sentinel-filled one-head oracle cache; every record its pages
    # hold and its sink/window rows must be byte-identical
    offs_h = offs.cpu().numpy()
    for b, h in ((0, 1), (37, 6), (63, 0)):
        L = int(p.lens[b])
        kb = k16[offs_h[b]:offs_h[b + 1], h:h + 1].cpu().numpy().view(np.uint16)
        vb = v16[offs_h[b]:offs_h[b + 1], h:h + 1].cpu().numpy().view(np.uint16)
        oc = O.Cache(p.num_pages, 1, w.batch, w.num_sink, w.window, fill=SENTINEL)
        oc.append(p.table[b], b, L - n_new, kb, vb, p.rot_k[h:h + 1], p.rot_v[h:h + 1],
                  w.clip, w.clip)
        pg = p.table[b, (L - n_new) // 16:(L + 15) // 16]
        gpu_rec = pm[torch.from_numpy(pg.astype(np.int64)).cuda(), h].cpu().numpy()
        nd_o = int((gpu_rec != oc.pages[pg, 0]).sum())
        _log(f"[append] full prefill, sequence {b} KV head {h}: {len(pg)} records, "
             f"{nd_o} bytes differ from the oracle")
        assert nd_o == 0
        assert np.array_equal(sm[b, h].cpu().numpy().view(np.uint16), oc.sinkwin[b, 0])


def test_full_prefill_shape_hadamard():
    """The Hadamard append at the full prefill shape, where each row slot of a wavefront takes
    many consecutive rows (sequence and page changes inside a slot's range): sampled (sequence,
    KV head) pairs against the oracle, every record and sink/window row byte for byte."""
    w, p, n_new, total, k16, v16, offs, start = _full_prefill_inputs()
    sk, sv = OF.hadamard_signs(70, w.num_kv_heads), OF.hadamard_signs(71, w.num_kv_heads)
    c = H.GpuCache(p, fill=SENTINEL)
    ops.rotate_quantize_append_hadamard(c.layout, c.pages, c.sinkwin, c.table, c.slots, k16, v16,
                                        offs, start, torch.from_numpy(sk).cuda(),
                                        torch.from_numpy(sv).cuda(), w.clip, w.clip)
    torch.cuda.synchronize()
    offs_h = offs.cpu().numpy()
    for b, h in ((0, 1), (37, 6), (63, 0)):
        L = int(p.lens[b])
        kb = k16[offs_h[b]:offs_h[b + 1], h:h + 1].cpu().numpy().view(np.uint16)
        vb = v16[offs_h[b]:offs_h[b + 1], h:h + 1].cpu().numpy().view(np.uint16)
        oc = O.Cache(p.num_pages, 1, w.batch, w.num_sink, w.window, fill=SENTINEL)
        oc.append(p.table[b], b, L - n_new, kb, vb, None, None, w.clip, w.clip,
                  hadamard_signs=(sk[h:h + 1], sv[h:h + 1]))
        pg = p.table[b, (L - n_new) // 16:(L + 15) // 16]
        gpu_rec = c.pages[torch.from_numpy(pg.astype(np.int64)).cuda(), h].cpu().numpy()
        nd_o = int((gpu_rec != oc.pages[pg, 0]).sum())
        _log(f"[append] full prefill (Hadamard), sequence {b} KV head {h}: {len(pg)} records, "
             f"{nd_o} bytes differ from the oracle")
        assert nd_o == 0
        assert np.array_equal(c.sinkwin[b, h].cpu().numpy().view(np.uint16), oc.sinkwin[b, 0])
