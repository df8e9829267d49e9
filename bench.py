"""Benchmark: one decode step of the rotated-INT2 mixed-precision paged attention on one GPU.

A step is one pass of the whole hot path over the batch: rotate-quantize-append of each
sequence's new token with the q rotation in the same launch (oscar_append_and_prepare), decode
attention (INT2 pages in equal per-worker runs, BF16 sink + window) and the combine of the
partials with R_V^T.  Default workload: Qwen3-8B-shaped layer, batch 64, 32 query / 8 KV heads,
head_dim 128, context lengths uniform in [16384, 32768], sink 4 + window 128 in BF16, INT2 bulk,
16-token pages, all inputs synthetic and already resident in HBM.

Prints ONE JSON line.  Extra fields: effective GB/s of the step, the decode-attention roofline
(bytes from the method's byte model / the launch's HIP-event duration), the prefill append of
2048 tokens per sequence, and the CPU oracle timed on a bounded sample of the same workload,
whose outputs are also compared with the GPU's for one (sequence, KV head) pair of every timed
INT2 workload.

Order of a run: cache fill; 20 decode steps after 1 s of idle (the cold-start figures: the
power management cuts the shader clock for the first ~10 ms of load); a step with a cache
scrub, a device copy and max(50, K) single steps with their own events (the spread: median,
p10, p90), which keep the load on; then, without an idle gap, the W warm-up steps and the K timed steps (the headline:
back-to-back decode steps as a serving loop runs them); the record-read probe; the prefill
timings; the INT2/BF16 comparisons; the CPU leg.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E peak
INT2_TOKEN_HEAD_BYTES = 96      # 32 B K codes + 32 B V codes + 16 B K meta + 16 B V meta
BF16_TOKEN_HEAD_BYTES = 512     # bf16 K + V rows
INT4_TOKEN_HEAD_BYTES = 160     # INT4 K + V codes (64 + 64) + K/V scale-zero (16 + 16)
METRIC = "decode attn tokens/s + effective HBM GB/s (% of peak), Qwen3-8B shape B=64 ctx=32k"


TRAFFIC_PROFILE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                               "int2_decode_qwen3_8b_b64_hbm_traffic.md")


def measured_traffic(workload: str):
    """HBM bytes per decode launch from the committed rocprofv3 counter summary, or None when
    that summary is for another workload or the decode kernels have changed since (their
    sources no longer hash to the recorded value)."""
    import hashlib
    try:
        text = open(TRAFFIC_PROFILE).read()
    except OSError:
        return None
    fields = {}
    for line in text.splitlines():
        if ":" in line:
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    try:
        if fields.get("workload") != workload:
            return None
        root = os.path.dirname(os.path.abspath(__file__))
        h = hashlib.sha256()
        for src in fields["kernel_sources"].split():
            h.update(open(os.path.join(root, src), "rb").read())
        if h.hexdigest() != fields["kernel_sources_sha256"]:
            return None
        return int(fields["traffic_bytes_per_launch"])
    except (KeyError, OSError, ValueError):
        return None


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def byte_model(w, lens):
    """Algorithmic HBM bytes of one decode step, split by part."""
    lens = np.asarray(lens, dtype=np.int64)
    n_sink = np.minimum(lens, w.num_sink)
    n_win = np.minimum(w.window, lens - n_sink)
    n_int2 = lens - n_sink - n_win
    hkv, hq, B = w.num_kv_heads, w.num_q_heads, w.batch
    int2 = int(hkv * INT2_TOKEN_HEAD_BYTES * n_int2.sum())
    bf16 = int(hkv * BF16_TOKEN_HEAD_BYTES * (n_sink + n_win).sum())
    q = B * hq * 128 * 2
    table = 4 * int(((lens + 15) // 16).sum())
    out = B * hq * 128 * 4
    # append of one token per sequence: bf16 K,V in; one INT2 slot + one bf16 window row out
    append = B * hkv * (2 * 128 * 2 + INT2_TOKEN_HEAD_BYTES + BF16_TOKEN_HEAD_BYTES)
    rot = 2 * hkv * 128 * 128 * 4
    return dict(int2=int2, bf16=bf16, q=q, table=table, out=out, append=append, rot=rot,
                decode_attention=int2 + bf16 + q + table,
                decode_kernel=int2 + bf16 + table,
                step=int2 + bf16 + q + table + out + append + rot)


def cpu_baseline(p, target_s: float):
    """The CPU oracle as it stands, on a bounded sample of the same workload: sequence 0, KV
    heads 0 and 1 (all G query heads of each), their oracle caches built untimed, then timed:
    repeated decode steps of one KV head (the append of the decoded token, which rewrites the
    same slot, plus decode attention) until about target_s seconds have been measured.  Scaled
    to one decode step of the sequence: tokens/s = 1 / (t_per_head * Hkv)."""
    from threadpoolctl import threadpool_limits
    from oracle import oscar_oracle as O
    from int2_rotated_kv_rotate_amd import workload as W
    import math

    w = p.w
    L = int(p.lens[0])
    G = w.group
    kb, vb = W.sequence_kv(w, 0, L)
    sm = float(np.float32(1.0 / math.sqrt(128.0)))
    heads = list(range(min(2, w.num_kv_heads)))
    per_step = []
    ref = {}
    with threadpool_limits(limits=1):
        caches = {}
        for h in heads:
            cache = O.Cache(p.num_pages, 1, 1, w.num_sink, w.window)
            cache.append(p.table[0], 0, 0, kb[:L - 1, h:h + 1], vb[:L - 1, h:h + 1],
                         p.rot_k[h:h + 1], p.rot_v[h:h + 1], w.clip, w.clip)
            caches[h] = cache
        while sum(per_step) < target_s:
            for h in heads:
                t0 = time.perf_counter()
                caches[h].append(p.table[0], 0, L - 1, kb[L - 1:, h:h + 1], vb[L - 1:, h:h + 1],
                                 p.rot_k[h:h + 1], p.rot_v[h:h + 1], w.clip, w.clip)
                ref[h] = O.decode_attention(caches[h], p.table[:1], np.zeros(1, np.int64),
                                            p.lens[:1], p.q[:1, h * G:(h + 1) * G],
                                            p.rot_k[h:h + 1], p.rot_v[h:h + 1], sm)
                per_step.append(time.perf_counter() - t0)
    t_head = float(np.mean(per_step))
    # bytes of one single-head decode step of this sequence by the method's byte model: its
    # INT2 records and BF16 sink/window rows, the G query rows and outputs, its table row
    n_sink = min(L, w.num_sink)
    n_win = min(w.window, L - n_sink)
    head_bytes = (INT2_TOKEN_HEAD_BYTES * (L - n_sink - n_win) + BF16_TOKEN_HEAD_BYTES *
                  (n_sink + n_win) + G * 128 * (2 + 4) + 4 * ((L + 15) // 16))
    return ref, {"value": 1.0 / (t_head * w.num_kv_heads), "unit": "tokens/s", "cores": 1,
            "effective_gbps": round(head_bytes / t_head / 1e9, 4),
            "kind": "oracle",
            "sample": (f"sequence 0 (L={L}), KV heads {heads} x {G} query heads: "
                       f"{len(per_step)} timed single-head decode steps (append of the new "
                       f"token + decode attention), {sum(per_step):.1f} s in total, scaled to "
                       f"all {w.num_kv_heads} KV heads of one decode step; one BLAS thread"),
            "host_cpus": os.cpu_count(), "affinity_cpus": len(os.sched_getaffinity(0)),
            "blas_threads": 1}


def oracle_pair(p, b: int, h: int, bits: int = 2):
    """The CPU oracle's decode of one (sequence, KV head) pair of a problem: its cache built by
    the same appends as the GPU run (the context, then the decoded token) and decode attention
    for the pair's query heads; bits 2 (INT2 records) or 4 (INT4).  Returns (out [G][128],
    lse [G])."""
    from oracle import oscar_oracle as O
    from int2_rotated_kv_rotate_amd import harness as H
    from int2_rotated_kv_rotate_amd import workload as W
    w = p.w
    L = int(p.lens[b])
    G = w.group
    kb, vb = W.sequence_kv(w, b, L, offsets=W.key_offsets(w), outliers=W.outlier_channels(w),
                           needle=W.needle_site(w, p.lens), q_bits=p.q)
    oc = O.Cache(p.num_pages, 1, w.batch, w.num_sink, w.window, bits=bits)
    args = (p.rot_k[h:h + 1], p.rot_v[h:h + 1], w.clip, w.clip)
    oc.append(p.table[b], b, 0, kb[:L - 1, h:h + 1], vb[:L - 1, h:h + 1], *args)
    oc.append(p.table[b], b, L - 1, kb[L - 1:, h:h + 1], vb[L - 1:, h:h + 1], *args)
    ref, ref_lse = O.decode_attention(oc, p.table[b:b + 1], np.array([b]), p.lens[b:b + 1],
                                      p.q[b:b + 1, h * G:(h + 1) * G], p.rot_k[h:h + 1],
                                      p.rot_v[h:h + 1], H.SM_SCALE)
    return ref[0], ref_lse[0]


def parity_record(out, lse, ref, ref_lse, **extra):
    """Per-row normwise error, elementwise error (floor: a quarter of the row's largest |ref|)
    and |dlse| of GPU rows against the oracle's, with the 2e-3 tolerance."""
    out = np.asarray(out, np.float64)
    row = float((np.abs(out - ref).max(-1) / np.abs(ref).max(-1)).max())
    el = float((np.abs(out - ref) / np.maximum(np.abs(ref),
                                               0.25 * np.abs(ref).max(-1, keepdims=True))).max())
    dl = float(np.abs(np.asarray(lse, np.float64) - ref_lse).max())
    return dict(extra, max_row_rel_err=row, max_elementwise_rel_err=el, max_abs_dlse=dl,
                tolerance=2e-3, ok=bool(row <= 2e-3 and el <= 2e-3 and dl <= 2e-3))


def time_scrubbed(fn, n: int, scrub):
    """Median (and p10, p90) of n launches of fn, each timed with an event pair on the current
    stream, with the whole last-level cache evicted before each launch by reading the 1 GiB
    scrub buffer (a read leaves clean lines: no write-backs land in the timed launch)."""
    import torch
    stream = torch.cuda.current_stream()
    ts = []
    sink = torch.empty((), dtype=scrub.dtype, device=scrub.device)
    for _ in range(n):
        torch.sum(scrub, dim=None, out=sink)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        fn()
        b.record(stream)
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b))
    ts = np.array(ts)
    return float(np.median(ts)), float(np.percentile(ts, 10)), float(np.percentile(ts, 90))


def record_read_probe(w, p, cache, stream):
    """The practical HBM ceiling of the decode launch's INT2 stream: the same records (every
    INT2 page of every (sequence, KV head) pair, in the decode kernel's order) read by
    oscar_read_records with the same number of wavefronts and none of the arithmetic."""
    import torch
    from int2_rotated_kv_rotate_amd import ops
    lens = np.asarray(p.lens, dtype=np.int64)
    ids = []
    for b, L in enumerate(lens):
        n_sink = min(L, w.num_sink)
        hi = L - min(w.window, L - n_sink)
        first, last = n_sink // 16, -(-hi // 16)
        if hi <= n_sink:
            continue
        pages = p.table[b, first:last].astype(np.int64)
        for h in range(w.num_kv_heads):
            ids.append(pages * w.num_kv_heads + h)
    ids = torch.from_numpy(np.concatenate(ids).astype(np.int32)).to(cache.device)
    workers = torch.cuda.get_device_properties(cache.device).multi_processor_count * 16
    out = torch.empty(64 * workers, dtype=torch.int32, device=cache.device)
    for _ in range(3):
        ops.read_records(cache.pages, ids, workers, out, stream)
    reps = 10
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    for a, b in ev:
        a.record(stream)
        ops.read_records(cache.pages, ids, workers, out, stream)
        b.record(stream)
    torch.cuda.synchronize()
    ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    nbytes = ids.numel() * INT2_TOKEN_HEAD_BYTES * 16
    gbps = nbytes / (ms / 1e3) / 1e9
    log(f"record-read probe: {ids.numel()} records, {ms:.4f} ms, {gbps:.0f} GB/s")
    return {"records": int(ids.numel()), "bytes": int(nbytes), "ms": round(ms, 5),
            "gbps": round(gbps, 1), "workers": workers,
            "what": "oscar_read_records over the decode launch's INT2 records in its order, "
                    "two 1536-byte records per step per wavefront, no arithmetic"}


def int2_vs_bf16(n_iter: int, samples: dict):
    """Attention (decode launch + combine) of the INT2 path against the BF16 paged baseline of
    the same library, with a 1 GiB cache scrub before every timed launch:
      * Qwen3-32B layer shape, context 32768: INT2 at batch 16 vs BF16 at batch 2 (about 1/8
        of the batch) and batch 3 (the equal-memory batch for 3 bits per element);
      * Qwen3-4B layer shape, batch 1, context 32768: latency of each;
      * long-context layer (32 query / 8 KV heads), batch 1, context 131072: latency of each;
      * the INT4 variant at the Qwen3-8B batch-64 shape (decode, and the prefill append of each
        sequence's last 2048 rows) and at the Qwen3-32B batch-16 shape.
    samples receives, per INT2 workload and for the INT4 one, the GPU outputs of one (sequence,
    KV head) pair for the oracle comparison of the CPU-baseline leg."""
    import torch
    from int2_rotated_kv_rotate_amd import harness as H
    from int2_rotated_kv_rotate_amd import ops
    from int2_rotated_kv_rotate_amd import workload as W

    scrub = torch.zeros(1 << 28, dtype=torch.float32, device="cuda")
    res = {}

    def attn_bytes(w, p, bf16):
        """Algorithmic bytes of one attention launch + combine (KV read, q, table, out)."""
        lens = np.asarray(p.lens, np.int64)
        hkv, hq, B = w.num_kv_heads, w.num_q_heads, w.batch
        if bf16:
            kv = hkv * BF16_TOKEN_HEAD_BYTES * int(lens.sum())
        else:
            n_sink = np.minimum(lens, w.num_sink)
            n_win = np.minimum(w.window, lens - n_sink)
            kv = hkv * (INT2_TOKEN_HEAD_BYTES * int((lens - n_sink - n_win).sum()) +
                        BF16_TOKEN_HEAD_BYTES * int((n_sink + n_win).sum()))
        return kv + B * hq * 128 * (2 + 4) + 4 * int(((lens + 15) // 16).sum())

    def int2_case(w):
        p = H.make_problem(w)
        cache = H.GpuCache(p)
        lk, lv = cache.fill_context()
        step = H.DecodeStep(cache)
        step.set_new_token(lk, lv)
        step.run()
        torch.cuda.synchronize()
        ms = time_scrubbed(step.attend, n_iter, scrub)
        g = H.capture_graph(step.attend)
        graph_ms = time_scrubbed(g.replay, n_iter, scrub)
        del g
        pool = p.num_pages * w.num_kv_heads * 1536
        # the outputs of one (sequence, KV head) pair, kept for the oracle comparison: the
        # longest sequence, the last KV head
        b = int(np.argmax(p.lens))
        h = w.num_kv_heads - 1
        G = w.group
        samples[w.name] = (p, b, h, step.out[b, h * G:(h + 1) * G].cpu().numpy(),
                           step.lse[b, h * G:(h + 1) * G].cpu().numpy(), 2)
        del step, cache
        return p, ms, pool, graph_ms

    def bf16_case(w):
        p = H.make_problem(w)
        bc = H.Bf16Cache(p)
        bc.attend()
        torch.cuda.synchronize()
        ms = time_scrubbed(bc.attend, n_iter, scrub)
        g = H.capture_graph(bc.attend)
        graph_ms = time_scrubbed(g.replay, n_iter, scrub)
        del g, bc
        pool = p.num_pages * w.num_kv_heads * 8192
        return p, ms, pool, graph_ms

    def gbps(w, p, ms, bf16):
        return round(attn_bytes(w, p, bf16) / (ms * 1e-3) / 1e9, 1)

    # Long context, batch 1 (131072 positions, the needle workload's cache): INT2 latency
    def graph_pair(gi, gb):
        """Latency of INT2 and BF16 attention replayed from HIP graphs (median, p10, p90)."""
        return {"int2_ms": round(gi[0], 4), "bf16_ms": round(gb[0], 4),
                "int2_ms_p10_p90": [round(gi[1], 4), round(gi[2], 4)],
                "bf16_ms_p10_p90": [round(gb[1], 4), round(gb[2], 4)],
                "latency_ratio": round(gb[0] / gi[0], 3)}

    wl = W.WORKLOADS["long_128k"]
    pl, (msl, _, _), _, gl = int2_case(wl)
    _, (msl_b, _, _), _, gl_b = bf16_case(wl)
    res["long_128k_b1"] = {"int2_ms": round(msl, 4), "bf16_ms": round(msl_b, 4),
                           "latency_ratio": round(msl_b / msl, 3),
                           "int2_effective_gbps": gbps(wl, pl, msl, False),
                           "bf16_effective_gbps": gbps(wl, pl, msl_b, True),
                           "graph": graph_pair(gl, gl_b)}
    log(f"long_128k B=1: INT2 {msl:.4f} ms, BF16 {msl_b:.4f} ms; from graphs INT2 "
        f"{gl[0]:.4f} ms, BF16 {gl_b[0]:.4f} ms")

    w32 = W.WORKLOADS["qwen3_32b"]
    p, (ms, p10, p90), pool, g32 = int2_case(w32)
    r32 = {"int2": {"batch": w32.batch, "ms": round(ms, 4), "tokens_per_s": round(w32.batch / ms * 1e3, 1),
                    "pool_bytes": pool, "effective_gbps": gbps(w32, p, ms, False),
                    "graph_ms": round(g32[0], 4)}}
    for bb in w32.bf16_batches:
        wb = W.scaled(w32, batch=bb, name=f"qwen3_32b_bf16_b{bb}")
        pb, (msb, _, _), poolb, _ = bf16_case(wb)
        r32[f"bf16_b{bb}"] = {"batch": bb, "ms": round(msb, 4),
                              "tokens_per_s": round(bb / msb * 1e3, 1), "pool_bytes": poolb,
                              "effective_gbps": gbps(wb, pb, msb, True)}
        r32[f"throughput_ratio_vs_bf16_b{bb}"] = round((w32.batch / ms) / (bb / msb), 3)
    res["qwen3_32b_ctx32k"] = r32
    log(f"qwen3_32b: INT2 B={w32.batch} {ms:.4f} ms; " + ", ".join(
        f"BF16 B={r32[k]['batch']} {r32[k]['ms']:.4f} ms" for k in r32 if k.startswith("bf16")))

    w4 = W.WORKLOADS["qwen3_4b"]
    p4, (ms_i, _, _), _, g4 = int2_case(w4)
    _, (ms_b, _, _), _, g4_b = bf16_case(w4)
    res["qwen3_4b_b1_ctx32k"] = {"int2_ms": round(ms_i, 4), "bf16_ms": round(ms_b, 4),
                                 "latency_ratio": round(ms_b / ms_i, 3),
                                 "int2_effective_gbps": gbps(w4, p4, ms_i, False),
                                 "bf16_effective_gbps": gbps(w4, p4, ms_b, True),
                                 "graph": graph_pair(g4, g4_b)}
    log(f"qwen3_4b B=1: INT2 {ms_i:.4f} ms, BF16 {ms_b:.4f} ms; from graphs INT2 "
        f"{g4[0]:.4f} ms, BF16 {g4_b[0]:.4f} ms")

    # The INT4 variant (2560-byte records, matrix-core decode) at the Qwen3-8B batch-64 shape
    w8 = W.WORKLOADS["qwen3_8b_b64"]
    p8 = H.make_problem(w8)
    c4 = H.GpuCache(p8, bits=4)
    lk, lv, tk4, tv4 = c4.fill_context(keep_tail=w8.prefill_new)
    st4 = H.DecodeStep(c4)
    st4.set_new_token(lk, lv)
    st4.run()
    torch.cuda.synchronize()
    ms4, _, _ = time_scrubbed(st4.attend, n_iter, scrub)
    # one (sequence, KV head) pair of the timed INT4 cache for the oracle comparison
    b4i, h4i, G8 = int(np.argmax(p8.lens)), w8.num_kv_heads - 1, w8.group
    samples["int4_" + w8.name] = (p8, b4i, h4i, st4.out[b4i, h4i * G8:(h4i + 1) * G8].cpu().numpy(),
                                  st4.lse[b4i, h4i * G8:(h4i + 1) * G8].cpu().numpy(), 4)
    lens = np.asarray(p8.lens, np.int64)
    n_sink = np.minimum(lens, w8.num_sink)
    n_win = np.minimum(w8.window, lens - n_sink)
    b4 = (w8.num_kv_heads * (INT4_TOKEN_HEAD_BYTES * int((lens - n_sink - n_win).sum()) +
                             BF16_TOKEN_HEAD_BYTES * int((n_sink + n_win).sum())) +
          w8.batch * w8.num_q_heads * 128 * (2 + 4) + 4 * int(((lens + 15) // 16).sum()))
    res["int4_qwen3_8b_b64"] = {"ms": round(ms4, 4), "tokens_per_s": round(w8.batch / ms4 * 1e3, 1),
                                "bytes": int(b4), "effective_gbps": round(b4 / (ms4 * 1e-3) / 1e9, 1),
                                "decode": "matrix cores: int8 logits, bf16 P.V, stream-K workers over "
                                          "2560-byte pages in a two-page LDS ring"}
    # The INT4 prefill append: each sequence's last prefill_new rows again (the same bytes),
    # one call, taken by the certified matrix-core kernel at this size
    offs4 = np.zeros(w8.batch + 1, dtype=np.int32)
    offs4[1:] = np.cumsum([t.shape[0] for t in tk4])
    kt4 = H.as_i16(np.concatenate(tk4)).cuda()
    vt4 = H.as_i16(np.concatenate(tv4)).cuda()
    offs4_d = torch.from_numpy(offs4).cuda()
    start4_d = torch.from_numpy(np.asarray([int(L) - 1 - t.shape[0] for L, t in zip(p8.lens, tk4)],
                                           dtype=np.int32)).cuda()

    def int4_prefill():
        ops.int4_rotate_quantize_append(c4.layout, c4.pages, c4.sinkwin, c4.table, c4.slots, kt4,
                                        vt4, offs4_d, start4_d, c4.rot_k, c4.rot_v, w8.clip,
                                        w8.clip)
    int4_prefill()
    torch.cuda.synchronize()
    a4, e4 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a4.record()
    for _ in range(3):
        int4_prefill()
    e4.record()
    torch.cuda.synchronize()
    pf4 = a4.elapsed_time(e4) / 3
    n4 = int(offs4[-1])
    res["int4_qwen3_8b_b64"]["prefill_append"] = {
        "tokens": n4, "ms": round(pf4, 4), "tokens_per_s": round(n4 / (pf4 / 1e3), 1),
        "rotation": "bf16 matrix cores, certified, uncertain values recomputed in fp64"}
    log(f"INT4 qwen3_8b B=64: {ms4:.4f} ms ({b4 / (ms4 * 1e-3) / 1e9:.0f} GB/s); prefill append "
        f"{n4} tokens {pf4:.3f} ms")
    del st4, c4, kt4, vt4

    # The INT4 variant at G = 8 (Qwen3-32B layer, batch 16, 32k): the matrix-core decode with
    # the (head, group pair) row layout
    wg8 = W.WORKLOADS["qwen3_32b"]
    pg8 = H.make_problem(wg8)
    c4g8 = H.GpuCache(pg8, bits=4)
    lk, lv = c4g8.fill_context()
    st4g8 = H.DecodeStep(c4g8)
    st4g8.set_new_token(lk, lv)
    st4g8.run()
    torch.cuda.synchronize()
    ms4g8, _, _ = time_scrubbed(st4g8.attend, n_iter, scrub)
    bg, hg, Gg = int(np.argmax(pg8.lens)), 0, wg8.group
    samples["int4_" + wg8.name] = (pg8, bg, hg, st4g8.out[bg, hg * Gg:(hg + 1) * Gg].cpu().numpy(),
                                   st4g8.lse[bg, hg * Gg:(hg + 1) * Gg].cpu().numpy(), 4)
    lens = np.asarray(pg8.lens, np.int64)
    n_sink = np.minimum(lens, wg8.num_sink)
    n_win = np.minimum(wg8.window, lens - n_sink)
    bg8 = (wg8.num_kv_heads * (INT4_TOKEN_HEAD_BYTES * int((lens - n_sink - n_win).sum()) +
                               BF16_TOKEN_HEAD_BYTES * int((n_sink + n_win).sum())) +
           wg8.batch * wg8.num_q_heads * 128 * (2 + 4) + 4 * int(((lens + 15) // 16).sum()))
    res["int4_qwen3_32b_b16"] = {"ms": round(ms4g8, 4),
                                 "tokens_per_s": round(wg8.batch / ms4g8 * 1e3, 1),
                                 "bytes": int(bg8),
                                 "effective_gbps": round(bg8 / (ms4g8 * 1e-3) / 1e9, 1),
                                 "decode": "matrix cores, G = 8: (head, group pair) rows, int8 "
                                           "logits, bf16 P.V"}
    log(f"INT4 qwen3_32b B=16: {ms4g8:.4f} ms ({bg8 / (ms4g8 * 1e-3) / 1e9:.0f} GB/s)")
    del st4g8, c4g8
    del scrub
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="qwen3_8b_b64")
    ap.add_argument("--workers", type=int, default=0,
                    help="INT2 worker wavefronts (0: one per resident slot of the device)")
    ap.add_argument("--max-splits", type=int, default=None,
                    help="INT2 partial slots per (sequence, KV head) (default: by batch size)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-compare", action="store_true",
                    help="skip the INT2 vs BF16 comparisons at the Qwen3-32B and batch-1 shapes")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one 1 GiB device copy (reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU (got --gpus {args.gpus}); this build has no "
              "multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    import torch
    from int2_rotated_kv_rotate_amd import harness as H
    from int2_rotated_kv_rotate_amd import ops
    from int2_rotated_kv_rotate_amd import workload as W

    ops.load_library()
    w = W.WORKLOADS[args.workload]
    p = H.make_problem(w)
    bm = byte_model(w, p.lens)
    log(f"workload {w.name}: B={w.batch} lens mean {p.lens.mean():.0f} "
        f"[{p.lens.min()}, {p.lens.max()}], pool {p.num_pages} pages "
        f"({p.num_pages * w.num_kv_heads * 1536 / 1e9:.2f} GB)")

    t0 = time.time()
    cache = H.GpuCache(p)
    tail = w.prefill_new if not args.no_prefill else 0
    if tail:
        last_k, last_v, tail_k, tail_v = cache.fill_context(keep_tail=tail)
    else:
        last_k, last_v = cache.fill_context()
    torch.cuda.synchronize()
    log(f"cache filled in {time.time() - t0:.1f} s")

    # The cache must be complete before decode is timed: append each sequence's last `tail`
    # tokens (the prefill workload) now; the same append is timed after the decode steps.
    if tail:
        offs = np.zeros(w.batch + 1, dtype=np.int32)
        offs[1:] = np.cumsum([t.shape[0] for t in tail_k])
        kt = H.as_i16(np.concatenate(tail_k)).cuda()
        vt = H.as_i16(np.concatenate(tail_v)).cuda()
        offs_d = torch.from_numpy(offs).cuda()
        start_d = torch.from_numpy((p.lens - 1 - tail).astype(np.int32)).cuda()

        kmean_d = torch.from_numpy(W.key_channel_means(w)).cuda()
        from int2_rotated_kv_rotate_amd import offline as OF
        signs_d = [torch.from_numpy(OF.hadamard_signs(seed, w.num_kv_heads)).cuda() for seed in (1, 2)]

        def do_prefill_hadamard():
            ops.rotate_quantize_append_hadamard(cache.layout, cache.pages, cache.sinkwin,
                                                cache.table, cache.slots, kt, vt, offs_d, start_d,
                                                signs_d[0], signs_d[1], w.clip, w.clip)

        def do_prefill(method=ops.APPEND_AUTO, k_mean=None):
            ops.rotate_quantize_append(cache.layout, cache.pages, cache.sinkwin, cache.table,
                                       cache.slots, kt, vt, offs_d, start_d, cache.rot_k,
                                       cache.rot_v, w.clip, w.clip, method=method, k_mean=k_mean)
        do_prefill()
        torch.cuda.synchronize()

    step = H.DecodeStep(cache, num_workers=args.workers, max_splits=args.max_splits)
    step.set_new_token(last_k, last_v)
    stream = torch.cuda.current_stream()

    def ev():
        return torch.cuda.Event(enable_timing=True)

    # The step on one stream: the new token's append and the query preparation in one launch
    # (oscar_append_and_prepare), the decode kernel (oscar_decode_attention_prepared) and the
    # combine; the same bytes and results as append + oscar_decode_attention + oscar_combine
    # (tests/test_gpu_fused_step.py).  The decode kernel, the dominant part, is bracketed by
    # events where it is timed.  (The append on a second stream beside the query preparation
    # was slower: each cross-stream join left the device idle for 7-18 us.)
    def timed_step(marks):
        a, b = ev(), ev()
        step.run_fused(before_decode=lambda: a.record(stream),
                       after_decode=lambda: b.record(stream))
        marks.append((a, b))

    # Cold start, for the record: after 1 s of idle the power management cuts the shader clock
    # for the first ~10 ms of load (measured with s_memtime against s_memrealtime: 2.4 GHz
    # idle, 1.3-1.6 GHz a few milliseconds into the load, ~2.1 GHz settled).  20 steps, the
    # decode kernel of each bracketed by events.
    step.run_fused()
    torch.cuda.synchronize()
    time.sleep(1.0)
    ca, cb = ev(), ev()
    cold_ev = []
    ca.record(stream)
    for _ in range(20):
        timed_step(cold_ev)
    cb.record(stream)
    torch.cuda.synchronize()
    cold_dec = np.array([a.elapsed_time(b) for a, b in cold_ev])
    cold = {"after_idle_s": 1.0, "steps": 20, "ms_per_step": round(ca.elapsed_time(cb) / 20, 5),
            "decode_launch_ms_mean": round(float(cold_dec.mean()), 5),
            "decode_launch_ms_max": round(float(cold_dec.max()), 5)}
    log(f"cold start (after 1 s idle): {cold}")

    # Before the timed region: the step with a cache scrub, the device copy and the spread of
    # single steps (memory-bound or decode work, which keeps the load on and lets the clock
    # settle); then, without an idle gap, the W warm-up steps and the K timed steps (the
    # headline: back-to-back decode steps as a serving loop runs them).  The record-read probe
    # and the prefill timings come after the timed region.
    scrub = torch.zeros(1 << 28, dtype=torch.float32, device="cuda")
    ms_scrub, _, _ = time_scrubbed(step.run_fused, max(5, args.steps // 2), scrub)
    # Achievable device-copy bandwidth in the same run: 1 GiB copied (2 GiB moved).
    csrc = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    cdst = torch.empty_like(csrc)
    cdst.copy_(csrc)
    c0, c1 = ev(), ev()
    torch.cuda.synchronize()
    c0.record(stream)
    for _ in range(5):
        cdst.copy_(csrc)
    c1.record(stream)
    torch.cuda.synchronize()
    copy_gbps = 2 * (1 << 30) / (c0.elapsed_time(c1) / 5 / 1e3) / 1e9
    del scrub, csrc, cdst
    log(f"step with cache scrub {ms_scrub:.4f} ms; device copy {copy_gbps:.0f} GB/s")
    # The spread of single steps: max(50, K) steps each bracketed by its own events (median,
    # p10, p90 over at least 50 iterations), run before the timed region so that their markers
    # do not touch the headline.
    n_spread = max(50, args.steps)
    sev = [ev() for _ in range(n_spread + 1)]
    sev[0].record(stream)
    for k in range(n_spread):
        step.run_fused()
        sev[k + 1].record(stream)
    torch.cuda.synchronize()
    step_ms = np.array([sev[k].elapsed_time(sev[k + 1]) for k in range(n_spread)])
    for _ in range(args.warmup):
        step.run_fused()
    torch.cuda.synchronize()

    # Timed region: exactly K whole steps back to back, bracketed by synchronisation.  The
    # decode kernel (the dominant part) is timed inside the same region, on its stream: an event
    # pair around the decode kernel of every 4th step (steps 1, 5, 9, ...), so that the samples
    # see the same clock and power state as the steps they belong to, while only a quarter of
    # the steps carry the two markers.
    start, end = ev(), ev()
    dec_ev = []
    start.record(stream)
    for k in range(args.steps):
        if k % 4 == 1:
            timed_step(dec_ev)
        else:
            step.run_fused()
    end.record(stream)
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(end) / args.steps
    if not dec_ev:  # fewer than 2 steps: one more step, timed on its own
        timed_step(dec_ev)
        torch.cuda.synchronize()
    attn_ms = np.array([a.elapsed_time(b) for a, b in dec_ev])
    attn_avg = float(attn_ms.mean())
    log(f"step {ms_step:.4f} ms; decode kernel avg {attn_avg:.4f} ms over {len(dec_ev)} timed "
        f"steps (min {attn_ms.min():.4f}, max {attn_ms.max():.4f}); single steps p10/p50/p90 "
        f"{np.percentile(step_ms, 10):.4f}/{np.percentile(step_ms, 50):.4f}/"
        f"{np.percentile(step_ms, 90):.4f} ms")

    record_read = record_read_probe(w, p, cache, stream)

    # The same step replayed from a HIP graph, the way a serving loop issues it when the
    # kernels are shorter than the host's work per launch (batch 1): K replays of the whole
    # step back to back, then K replays of the decode launch alone (q preparation + decode
    # kernel), each bracketed by events.  After the timed region: not part of the headline.
    g_step = H.capture_graph(step.run_fused)
    g_dec = H.capture_graph(step.decode_only)
    n_rep = max(args.steps, 5)
    ga, gb = ev(), ev()
    ga.record(stream)
    for _ in range(n_rep):
        g_step.replay()
    gb.record(stream)
    dev_ev = [ev() for _ in range(n_rep + 1)]
    dev_ev[0].record(stream)
    for k in range(n_rep):
        g_dec.replay()
        dev_ev[k + 1].record(stream)
    torch.cuda.synchronize()
    graph = {"replays": n_rep, "ms_per_step": round(ga.elapsed_time(gb) / n_rep, 5),
             "decode_launch_ms": round(float(np.mean(
                 [dev_ev[k].elapsed_time(dev_ev[k + 1]) for k in range(n_rep)])), 5)}
    del g_step, g_dec
    log(f"graph replay: step {graph['ms_per_step']:.4f} ms, decode launch "
        f"{graph['decode_launch_ms']:.4f} ms")
    prefill = None
    if tail:
        # Both append kernels write the same bytes; the automatic choice for this size is the
        # matrix-core one, and the fp64 vector kernel is timed beside it.
        reps = 3
        pf = {}
        cases = (("matrix", lambda: do_prefill(ops.APPEND_MATRIX)),
                 ("vector", lambda: do_prefill(ops.APPEND_VECTOR)),
                 ("matrix_key_mean", lambda: do_prefill(ops.APPEND_MATRIX, kmean_d)),
                 ("hadamard", do_prefill_hadamard))
        for name, fn in cases:
            fn()
            a, b = ev(), ev()
            a.record(stream)
            for _ in range(reps):
                fn()
            b.record(stream)
            torch.cuda.synchronize()
            pf[name] = a.elapsed_time(b) / reps
        pf_ms = pf["matrix"]
        n_new = int(offs[-1])
        pf_bytes = n_new * w.num_kv_heads * (2 * 256 + INT2_TOKEN_HEAD_BYTES) + \
            w.batch * w.num_kv_heads * w.window * BF16_TOKEN_HEAD_BYTES + bm["rot"]
        prefill = {"tokens": n_new, "ms": round(pf_ms, 4),
                   "tokens_per_s": round(n_new / (pf_ms / 1e3), 1),
                   "effective_gbps": round(pf_bytes / (pf_ms / 1e3) / 1e9, 1),
                   "rotation": "bf16 matrix cores, certified, uncertain values recomputed in fp64",
                   "fp64_vector_kernel_ms": round(pf["vector"], 4),
                   "with_key_mean_ms": round(pf["matrix_key_mean"], 4),
                   "hadamard_rotation_ms": round(pf["hadamard"], 4),
                   "hadamard_effective_gbps": round(pf_bytes / (pf["hadamard"] / 1e3) / 1e9, 1)}
        log(f"prefill append {n_new} tokens: matrix cores {pf_ms:.3f} ms, fp64 vector "
            f"{pf['vector']:.3f} ms, matrix cores with a key mean {pf['matrix_key_mean']:.3f} ms, "
            f"Hadamard rotation {pf['hadamard']:.3f} ms")
        do_prefill(ops.APPEND_MATRIX)  # the cache without the key mean again
        step.run()  # restore the window rows the prefill re-append rewrote
        torch.cuda.synchronize()

    tokens_per_s = w.batch / (ms_step / 1e3)
    step_gbps = bm["step"] / (ms_step / 1e3) / 1e9
    attn_gbps = bm["decode_kernel"] / (attn_avg / 1e3) / 1e9

    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log("copy calibration: 1 GiB device copy done")

    gpu_out = step.out.cpu().numpy()
    gpu_lse = step.lse.cpu().numpy()
    samples = {}
    compare = None
    if not args.no_compare:
        compare = int2_vs_bf16(20, samples)

    # CPU leg: the oracle timed on a bounded sample of the headline workload (the CPU
    # baseline), and the oracle's outputs of one (sequence, KV head) pair of every timed INT2
    # and INT4 workload compared with the GPU's.
    cpu = None
    parity = None
    if not args.no_cpu:
        t0 = time.time()
        ref, cpu = cpu_baseline(p, args.cpu_seconds)
        log(f"cpu oracle baseline: {cpu['value']:.4f} tokens/s ({time.time() - t0:.1f} s)")
        G = w.group
        outs = [gpu_out[0, h * G:(h + 1) * G] for h in sorted(ref)]
        lses = [gpu_lse[0, h * G:(h + 1) * G] for h in sorted(ref)]
        parity = {w.name: parity_record(np.stack(outs), np.stack(lses),
                                        np.stack([ref[h][0][0] for h in sorted(ref)]),
                                        np.stack([ref[h][1][0] for h in sorted(ref)]),
                                        sequence=0, kv_heads=sorted(ref))}
        for name, (pp, b, h, o, l, bits) in samples.items():
            t1 = time.time()
            r, rl = oracle_pair(pp, b, h, bits)
            parity[name] = parity_record(o, l, r, rl, sequence=b, kv_heads=[h],
                                         context=int(pp.lens[b]))
            log(f"parity {name}: {parity[name]} ({time.time() - t1:.1f} s)")
        log(f"parity {w.name}: {parity[w.name]}")

    line = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int2-kv/int8+bf16-mfma/fp32-acc",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "q_heads": w.num_q_heads,
                   "kv_heads": w.num_kv_heads, "head_dim": 128,
                   "ctx": f"U[{w.ctx_min},{w.ctx}]" if w.ctx_min else w.ctx,
                   "mean_ctx": float(p.lens.mean()), "sink": w.num_sink, "window": w.window,
                   "page": 16, "workers": args.workers or "auto",
                   "max_splits": step.max_splits},
        "effective_gbps": round(step_gbps, 1),
        "pct_of_peak": round(100.0 * step_gbps / HBM_PEAK_GBPS, 2),
        "kv_positions_per_s": round(float(np.asarray(p.lens, np.int64).sum()) / (ms_step / 1e3), 1),
        "step_ms_p10_p50_p90": [round(float(np.percentile(step_ms, q)), 5) for q in (10, 50, 90)],
        "step_spread_samples": int(len(step_ms)),
        "cold_start": cold,
        "ms_per_step_cache_scrubbed": round(ms_scrub, 5),
        "copy_gbps": round(copy_gbps, 1),
        "roofline": {"bound": "hbm", "kernel": "int2_decode_kernel (INT2 runs + BF16 sink/window, "
                     "oscar_decode_attention_prepared; q prepared by oscar_append_and_prepare)",
                     "achieved": round(attn_gbps, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(attn_gbps / HBM_PEAK_GBPS, 4),
                     "bytes_per_launch": bm["decode_kernel"], "launch_ms": round(attn_avg, 5),
                     "launch_samples": len(dec_ev),
                     "launch_ms_p10_p90": [round(float(np.percentile(attn_ms, q)), 5) for q in (10, 90)],
                     "traffic": measured_traffic(w.name),
                     "frac_of_copy": round(attn_gbps / copy_gbps, 4),
                     "frac_of_record_read": round(attn_gbps / record_read["gbps"], 4)},
        "record_read": record_read,
        "graph_replay": graph,
        "bytes": bm,
        "prefill_append": prefill,
        "cpu_baseline": cpu,
        "parity": parity,
        "int2_vs_bf16": compare,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
