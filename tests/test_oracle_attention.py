"""Pins of the oracle's cache model, attention and split merge (CPU only).

Closed forms and invariants: rotation invariance of unquantised attention, single-token and
zero-query special cases, a short context that never touches INT2, block-table permutation
invariance, the sink/window placement rule, and partition invariance of the split merge.
"""
import math

import numpy as np
import pytest
from scipy.special import logsumexp

from oracle import oscar_oracle as O
from int2_rotated_kv_rotate_amd import workload as W

SM = float(np.float32(1.0 / math.sqrt(128.0)))


def test_attention_is_invariant_under_the_rotation():
    """softmax(qR (KR)^T) (VR) R^T == softmax(q K^T) V for orthogonal R (fp64, 1e-12)."""
    rng = np.random.default_rng(11)
    R = W.rotations(W.WORKLOADS["qwen3_4b"], "k")[3]
    q = rng.standard_normal(128) * 2
    k = rng.standard_normal((300, 128)) * 3
    v = rng.standard_normal((300, 128))
    o0, l0, a0 = O.softmax_attention(q, k, v, SM)
    o1, l1, a1 = O.softmax_attention(q @ R, k @ R, v @ R, SM)
    assert np.abs(o1 @ R.T - o0).max() <= 1e-12 * max(1.0, np.abs(o0).max())
    assert abs(l1 - l0) <= 1e-12 * abs(l0)
    assert np.abs(a1 - a0).max() <= 1e-13


def test_attention_matches_logsumexp_form():
    rng = np.random.default_rng(12)
    q = rng.standard_normal(128)
    k = rng.standard_normal((77, 128)) * 4
    v = rng.standard_normal((77, 128))
    o, lse, a = O.softmax_attention(q, k, v, SM)
    z = np.float32(SM) * (k @ q)
    assert abs(lse - logsumexp(z)) <= 1e-12 * abs(lse)
    ref = (np.exp(z - logsumexp(z))[:, None] * v).sum(0)
    assert np.abs(o - ref).max() <= 1e-13
    assert abs(a.sum() - 1.0) <= 1e-14


def test_attention_special_cases():
    rng = np.random.default_rng(13)
    v = rng.standard_normal((40, 128))
    k = rng.standard_normal((40, 128))
    o, _, _ = O.softmax_attention(rng.standard_normal(128), k[:1], v[:1], SM)
    assert np.array_equal(o, v[0])
    o, lse, a = O.softmax_attention(np.zeros(128), k, v, SM)
    assert np.allclose(o, v.mean(0), atol=1e-14) and abs(lse - math.log(40)) < 1e-14


def _tiny_cache(w, lens, fill=0, table_seed_shift=0, extra=4):
    table, npages = W.block_table(w, lens, extra_pages=extra)
    if table_seed_shift:
        rng = np.random.default_rng(table_seed_shift)
        perm = rng.permutation(npages).astype(np.int32)
        table = np.where(table >= 0, perm[np.maximum(table, 0)], -1).astype(np.int32)
    cache = O.Cache(npages, w.num_kv_heads, w.batch, w.num_sink, w.window, fill=fill)
    return cache, table


def _fill(cache, table, w, lens, Rk, Rv, chunks=(None,)):
    q = W.queries(w)
    for b in range(w.batch):
        kb, vb = W.sequence_kv(w, b, int(lens[b]))
        L = int(lens[b])
        cuts = [0] + [c for c in chunks if c is not None and 0 < c < L] + [L]
        for t0, t1 in zip(cuts[:-1], cuts[1:]):
            cache.append(table[b], b, t0, kb[t0:t1], vb[t0:t1], Rk, Rv, w.clip, w.clip)
    return q


def test_short_context_is_plain_bf16_attention_of_rotated_rows():
    """L <= S + W: no INT2 read; equals attention over bf16(x R) with q R_K and R_V^T."""
    w = W.scaled(W.WORKLOADS["tiny"], ctx=60)
    lens = W.seq_lengths(w)
    Rk = W.rotations(w, "k").astype(np.float32)
    Rv = W.rotations(w, "v").astype(np.float32)
    cache, table = _tiny_cache(w, lens)
    q = _fill(cache, table, w, lens, Rk, Rv)
    out, lse = O.decode_attention(cache, table, np.arange(w.batch), lens, q, Rk, Rv, SM)
    kb, vb = W.sequence_kv(w, 0, 60)
    yk = O.rotate_rows(kb[:, 0], Rk[0])
    yv = O.rotate_rows(vb[:, 0], Rv[0])
    kr = O.bf16_bits_to_f64(O.f32_to_bf16_bits(yk))
    vr = O.bf16_bits_to_f64(O.f32_to_bf16_bits(yv))
    qr = W.bf16_bits_to_f32(q[0, 0]).astype(np.float64) @ Rk[0].astype(np.float64)
    o, l, _ = O.softmax_attention(qr, kr, vr, SM)
    assert np.abs(out[0, 0] - o @ Rv[0].astype(np.float64).T).max() <= 1e-12
    assert abs(lse[0, 0] - l) <= 1e-12


def test_read_sequence_mixes_bf16_and_int2_as_defined():
    w = W.WORKLOADS["tiny"]
    lens = W.seq_lengths(w)
    L = int(lens[0])
    Rk = W.rotations(w, "k").astype(np.float32)
    Rv = W.rotations(w, "v").astype(np.float32)
    cache, table = _tiny_cache(w, lens)
    _fill(cache, table, w, lens, Rk, Rv, chunks=(100, 300, L - 1))
    k, v, is_int2 = cache.read_sequence(table[0], 0, 0, L)
    S, Wn = w.num_sink, w.window
    assert not is_int2[:S].any() and not is_int2[L - Wn:].any() and is_int2[S:L - Wn].all()
    kb, vb = W.sequence_kv(w, 0, L)
    yk, kc, ks, kz = O.quantize_rows(kb[:, 0], Rk[0], w.clip)
    yv, vc, vs, vz = O.quantize_rows(vb[:, 0], Rv[0], w.clip)
    bulk = np.arange(S, L - Wn)
    assert np.array_equal(k[bulk], O.dequant(kc, ks, kz)[bulk])
    assert np.array_equal(v[bulk], O.dequant(vc, vs, vz)[bulk])
    bf = np.r_[np.arange(S), np.arange(L - Wn, L)]
    assert np.array_equal(k[bf], O.bf16_bits_to_f64(O.f32_to_bf16_bits(yk[bf])))
    assert np.array_equal(v[bf], O.bf16_bits_to_f64(O.f32_to_bf16_bits(yv[bf])))
    # on average the reconstruction error is well under half a quantisation step
    yh = O.dequant(kc, ks, kz)
    step = np.repeat(ks.astype(np.float64), 32, axis=1)
    assert np.abs(yh - yk).mean() < 0.5 * step.mean()


def test_chunked_appends_equal_one_append_and_permutation_invariance():
    w = W.scaled(W.WORKLOADS["qwen3_4b"], ctx=300)
    w = W.scaled(w, batch=2, ctx=300, ctx_min=200)
    lens = W.seq_lengths(w)
    Rk = W.rotations(w, "k").astype(np.float32)
    Rv = W.rotations(w, "v").astype(np.float32)
    c1, t1 = _tiny_cache(w, lens)
    q = _fill(c1, t1, w, lens, Rk, Rv)
    c2, t2 = _tiny_cache(w, lens, table_seed_shift=77)
    _fill(c2, t2, w, lens, Rk, Rv, chunks=(17, 130, 131))
    for b in range(2):
        for h in range(w.num_kv_heads):
            a = c1.read_sequence(t1[b], b, h, int(lens[b]))
            bb = c2.read_sequence(t2[b], b, h, int(lens[b]))
            assert np.array_equal(a[0], bb[0]) and np.array_equal(a[1], bb[1])
    o1, l1 = O.decode_attention(c1, t1, np.arange(2), lens, q, Rk, Rv, SM)
    o2, l2 = O.decode_attention(c2, t2, np.arange(2), lens, q, Rk, Rv, SM)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_sink_window_rule():
    S, Wn = 4, 8
    assert [O.sink_window_index(p, S, Wn, 30) for p in range(4)] == [0, 1, 2, 3]
    assert O.sink_window_index(21, S, Wn, 30) is None
    assert O.sink_window_index(22, S, Wn, 30) == S + 22 % Wn
    assert O.sink_window_index(29, S, Wn, 30) == S + 29 % Wn
    rows = {O.sink_window_index(p, S, Wn, 30) for p in range(22, 30)}
    assert rows == set(range(S, S + Wn))


def _level_rows(rng, n):
    """Rows whose every 32-channel group lies exactly on 4 evenly spaced levels (both ends hit)."""
    x = np.empty((n, 128), np.float32)
    for i in range(n):
        for g in range(4):
            a = rng.choice([-3.0, -2.0, -1.5, -0.75, 0.5])
            d = rng.choice([0.25, 0.5, 1.0, 2.0])
            k = rng.integers(0, 4, 32)
            k[rng.choice(32, 2, replace=False)] = [0, 3]
            x[i, 32 * g:32 * g + 32] = a + d * k
    return W.to_bf16_bits(x)


def test_int2_path_is_exact_on_level_aligned_rows():
    """With R = I, clip = 1 and rows lying on 4 levels per group, INT2 reconstructs the rows
    exactly, so decode attention over the mixed cache equals plain attention over the rows."""
    rng = np.random.default_rng(15)
    L, S, Wn, hkv, hq = 200, 4, 16, 2, 4
    kb = np.stack([_level_rows(rng, L) for _ in range(hkv)], axis=1)
    vb = np.stack([_level_rows(rng, L) for _ in range(hkv)], axis=1)
    eye = np.stack([np.eye(128, dtype=np.float32)] * hkv)
    table = np.array([rng.permutation(20)[:13]], np.int32)
    cache = O.Cache(20, hkv, 1, S, Wn)
    cache.append(table[0], 0, 0, kb[:120], vb[:120], eye, eye, 1.0, 1.0)
    cache.append(table[0], 0, 120, kb[120:], vb[120:], eye, eye, 1.0, 1.0)
    q = W.to_bf16_bits(rng.standard_normal((1, hq, 128)).astype(np.float32) * 0.3)
    out, lse = O.decode_attention(cache, table, [0], [L], q, eye, eye, SM)
    for j in range(hq):
        h = j // 2
        k, v, is_int2 = cache.read_sequence(table[0], 0, h, L)
        assert is_int2.sum() == L - S - Wn
        assert np.array_equal(k, W.bf16_bits_to_f32(kb[:, h]).astype(np.float64))
        assert np.array_equal(v, W.bf16_bits_to_f32(vb[:, h]).astype(np.float64))
        o, l, _ = O.softmax_attention(W.bf16_bits_to_f32(q[0, j]).astype(np.float64),
                                      W.bf16_bits_to_f32(kb[:, h]).astype(np.float64),
                                      W.bf16_bits_to_f32(vb[:, h]).astype(np.float64), SM)
        assert np.abs(out[0, j] - o).max() <= 1e-13 and abs(lse[0, j] - l) <= 1e-12


@pytest.mark.parametrize("nsplit", [1, 2, 5, 17])
def test_merge_of_any_partition_equals_single_softmax(nsplit):
    rng = np.random.default_rng(100 + nsplit)
    n = 200
    z = rng.standard_normal(n) * 6          # natural-log logits
    v = rng.standard_normal((n, 128))
    cuts = np.sort(rng.choice(np.arange(1, n), nsplit - 1, replace=False)) if nsplit > 1 else []
    parts = np.split(np.arange(n), cuts)
    m2, l, o = [], [], []
    for idx in parts:
        z2 = z[idx] * math.log2(math.e)
        m = z2.max()
        e = np.exp2(z2 - m)
        m2.append(m)
        l.append(e.sum())
        o.append(e @ v[idx])
    # an empty split must be ignored
    m2.append(-np.inf)
    l.append(0.0)
    o.append(np.zeros(128))
    ot, lse = O.merge_partials(np.array(m2), np.array(l), np.array(o))
    ref = np.exp(z - logsumexp(z)) @ v
    assert np.abs(ot - ref).max() <= 1e-12
    assert abs(lse - logsumexp(z)) <= 1e-12 * abs(logsumexp(z))


def test_bf16_page_layout_and_baseline_attention():
    rng = np.random.default_rng(14)
    page = np.zeros(O.BF16_PAGE_ELEMS, np.uint16)
    kr = [W.to_bf16_bits(rng.standard_normal(128).astype(np.float32)) for _ in range(16)]
    vr = [W.to_bf16_bits(rng.standard_normal(128).astype(np.float32)) for _ in range(16)]
    for r in range(16):
        O.bf16_write_token(page, r, kr[r], vr[r])
    k, v = O.bf16_read_page(page)
    assert np.array_equal(k, np.stack(kr)) and np.array_equal(v, np.stack(vr))
    # V is stored channel-major: element (c, r) at 2048 + 16 c + r
    assert page[2048 + 16 * 5 + 3] == vr[3][5]
    # baseline attention over pages equals plain attention over the same rows
    L = 37
    kb = W.to_bf16_bits(rng.standard_normal((L, 2, 128)).astype(np.float32))
    vb = W.to_bf16_bits(rng.standard_normal((L, 2, 128)).astype(np.float32))
    pages = np.zeros((5, 2, O.BF16_PAGE_ELEMS), np.uint16)
    table = np.array([[4, 0, 2]], np.int32)
    for p in range(L):
        for h in range(2):
            O.bf16_write_token(pages[table[0, p // 16], h], p % 16, kb[p, h], vb[p, h])
    q = W.to_bf16_bits(rng.standard_normal((1, 4, 128)).astype(np.float32))
    out, lse = O.bf16_decode_attention(pages, table, [L], q, SM, 2)
    for j in range(4):
        h = j // 2
        o, l, _ = O.softmax_attention(W.bf16_bits_to_f32(q[0, j]).astype(np.float64),
                                      W.bf16_bits_to_f32(kb[:, h]).astype(np.float64),
                                      W.bf16_bits_to_f32(vb[:, h]).astype(np.float64), SM)
        assert np.abs(out[0, j] - o).max() <= 1e-14 and abs(lse[0, j] - l) <= 1e-12
