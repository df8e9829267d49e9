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


@pytest.mark.parametrize("with_mean", [False, True])
def test_int4_prefill_shape_matrix_vs_vector(with_mean):
    """The INT4 append at the benchmark's prefill shape (64 sequences x 2048 new tokens at the end
    of 16K-32K contexts, workload-recipe rows drawn on the GPU): one call (the matrix-core kernel,
    from 256 rows on) against the same rows appended in calls of at most 255 rows (the fp64
    vector kernel), every page and sink/window byte; plain and with the key mean."""
    from int2_rotated_kv_rotate_amd import ops
    w = W.WORKLOADS["qwen3_8b_b64"]
    p = H.make_problem(w)
    n_new = w.prefill_new
    gen = torch.Generator(device="cuda")
    gen.manual_seed(4096)
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
    del k, v
    offs = torch.arange(0, total + 1, n_new, dtype=torch.int32, device="cuda")
    start = torch.from_numpy((p.lens - n_new).astype(np.int32)).cuda()
    k_mean = torch.from_numpy(W.key_channel_means(w)).cuda() if with_mean else None
    one = H.GpuCache(p, fill=SENTINEL, bits=4)
    ops.int4_rotate_quantize_append(one.layout, one.pages, one.sinkwin, one.table, one.slots, k16,
                                    v16, offs, start, one.rot_k, one.rot_v, w.clip, w.clip,
                                    k_mean=k_mean)
    torch.cuda.synchronize()
    chunked = H.GpuCache(p, fill=SENTINEL, bits=4)
    chunk = 255
    B = w.batch
    for b in range(B):
        for c0 in range(0, n_new, chunk):
            n = min(chunk, n_new - c0)
            o = np.zeros(B + 1, np.int32)
            o[b + 1:] = n
            sp = (p.lens - n_new).astype(np.int32)
            sp[b] += c0
            r0 = b * n_new + c0
            ops.int4_rotate_quantize_append(chunked.layout, chunked.pages, chunked.sinkwin,
                                            chunked.table, chunked.slots,
                                            k16[r0:r0 + n].contiguous(), v16[r0:r0 + n].contiguous(),
                                            torch.from_numpy(o).cuda(), torch.from_numpy(sp).cuda(),
                                            chunked.rot_k, chunked.rot_v, w.clip, w.clip,
                                            k_mean=k_mean)
    torch.cuda.synchronize()
    nd = int((one.pages != chunked.pages).sum().item())
    ns = int((one.sinkwin != chunked.sinkwin).sum().item())
    _log(f"[int4] prefill shape {total} rows (key mean {with_mean}): {nd} page bytes, "
         f"{ns} sink/window entries differ between the matrix-core and vector kernels")
    assert nd == 0 and ns == 0
    # and the new rows really were written (the sentinel replaced in a tail record)
    last_page = int(p.table[0, (int(p.lens[0]) - 1) // 16])
    assert not bool((one.pages[last_page, 0, :1024] == SENTINEL).all().item())


@pytest.mark.parametrize("kind", ["special_rows", "symmetric_groups"])
def test_int4_matrix_append_special_rows(kind):
    """Rows that stress the matrix-core append's certification, in INT4 records (whole contexts,
    so every call takes the matrix-core kernel and writes sink, window and bulk rows), against the
    oracle byte for byte: rows along a column of R, zeros, subnormals and mixed 2^-20 / 2^8
    magnitudes; or, under the identity rotation, groups with max = -min (a 16-level code
    threshold exactly at a grid point), one-signed and constant groups."""
    w = W.scaled(W.WORKLOADS["qwen3_4b"], name="int4_" + kind, batch=2, ctx=700, ctx_min=400)
    rng = np.random.default_rng(77)
    if kind == "special_rows":
        from test_gpu_append_methods import _special_rows
        p = H.make_problem(w)
        ks = [_special_rows(rng, p.rot_k, int(L)) for L in p.lens]
        vs = [_special_rows(rng, p.rot_v, int(L)) for L in p.lens]
    else:
        eye = np.broadcast_to(np.eye(128), (w.num_kv_heads, 128, 128)).copy()
        p = H.make_problem(w, rot_k=eye, rot_v=eye)

        def rows(n):
            x = rng.uniform(-1.0, 1.0, size=(n, w.num_kv_heads, 4, 32)).astype(np.float32)
            a = np.float32(2.0) ** rng.integers(-8, 8, size=(n, w.num_kv_heads, 4, 1)).astype(np.float32)
            x *= a
            kk = rng.integers(0, 4, size=(n, w.num_kv_heads, 4))
            x[..., 0] = np.where(kk < 2, a[..., 0], x[..., 0])
            x[..., 1] = np.where(kk < 2, -a[..., 0], x[..., 1])
            x = np.where((kk == 2)[..., None], np.abs(x), x)
            x = np.where((kk == 3)[..., None], a, x)
            return W.to_bf16_bits(x.reshape(n, w.num_kv_heads, 128))

        ks = [rows(int(L)) for L in p.lens]
        vs = [rows(int(L)) for L in p.lens]
    c = H.GpuCache(p, fill=SENTINEL, bits=4)
    c.append(ks, vs, [0] * w.batch)
    torch.cuda.synchronize()
    oc = O.Cache(p.num_pages, w.num_kv_heads, w.batch, w.num_sink, w.window, fill=SENTINEL, bits=4)
    for b in range(w.batch):
        oc.append(p.table[b], b, 0, ks[b], vs[b], p.rot_k, p.rot_v, w.clip, w.clip)
    nd = int((c.pages.cpu().numpy() != oc.pages).sum())
    _log(f"[int4] matrix append {kind}: {sum(k.shape[0] for k in ks)} rows, {nd} page bytes differ")
    assert nd == 0
    assert np.array_equal(c.sinkwin.cpu().numpy().view(np.uint16), oc.sinkwin)
