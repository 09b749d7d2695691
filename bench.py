#!/usr/bin/env python3
"""Benchmark of compressed decode attention on one MI355X.

A step is one decode-attention call over a compressed store (query rotation, score estimate over every stored
key, top-T selection, exact sparse attention, output rotation) for one layer of the workload.  The store is
built once per run by the library's compression call, which is timed as its own leg and reported under
"compress".  The printed JSON line reports context tokens per second (sum of the requests' contexts divided by
the step time), the roofline of the dominant kernel (the score gather-dot, HBM-bound) from HIP events recorded
around its launches in the first quarter of the timed region, and the CPU oracle timed on a bounded sample of the
same workload.
The other workloads of the target (one 1048576-token request, the 16-request ragged mix) and the single-layer
Llama-3.1-8B shape are measured with the same compress and decode legs and reported under "workloads", each with
the uncompressed baseline on its inputs.

Usage: python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--workload batch8_128k] [--cpu-seconds 12]
                       [--extras million,ragged16,llama_layer]
"""
from __future__ import annotations

import argparse
import gc
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402

HBM_PEAK_GBPS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0
METRIC = "compressed decode-attn context tokens/s per layer; achieved HBM GB/s vs peak"
# sources whose hash a counter summary in profiles/ must carry to be used (the kernel and its shared header)
KERNEL_SOURCES = {
    "score": ["kv_cache_compression_svd_amd/csrc/decode.hip", "kv_cache_compression_svd_amd/csrc/common.cuh"],
    "dense_attend": ["kv_cache_compression_svd_amd/csrc/dense.hip", "kv_cache_compression_svd_amd/csrc/common.cuh"],
    "gram": ["kv_cache_compression_svd_amd/csrc/gram.hip", "kv_cache_compression_svd_amd/csrc/common.cuh"],
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="batch8_128k", choices=W.ORDER)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--workers", type=int, default=min(16, os.cpu_count() or 1))
    ap.add_argument("--no-layers", dest="layers", action="store_false",
                    help="skip the layer-batched extra (32 layers x 32768 tokens in one call)")
    ap.add_argument("--no-pool", dest="pool", action="store_false",
                    help="skip the paged-pool extra (the same requests added to a pool, decoded through a view)")
    ap.add_argument("--extras", default="million,ragged16,llama_layer",
                    help="other workloads measured with the same compress and decode legs (comma list, '' for none)")
    return ap.parse_args()


def source_hash(kernel: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def read_traffic(kernel: str, workload: str):
    """HBM bytes per launch of a kernel from the committed rocprofv3 counter summary, when it was taken on the
    current kernel source; otherwise None."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_pmc.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("source_sha256_16") != source_hash(kernel):
        return None
    try:
        return float(vals["traffic_bytes_per_dispatch"])
    except (KeyError, ValueError):
        return None


def store_bytes(codes: np.ndarray, cu, Hkv: int, keep, bv: int):
    """Per-segment payload sizes of both tensors from the strategy codes: (K sizes, V sizes, n_s per segment)."""
    n = np.diff(np.asarray(cu, dtype=np.int64))
    S_r = (n + 63) // 64
    S = int(S_r.sum()) * Hkv
    ns = np.zeros(S, dtype=np.int64)
    pos = 0
    for r in range(len(n)):
        seg = np.minimum(64, n[r] - 64 * np.arange(S_r[r]))
        for _ in range(Hkv):
            ns[pos:pos + S_r[r]] = seg
            pos += S_r[r]
    keep = np.asarray(keep)
    c = keep[codes.astype(np.int64)]
    row = c * (bv + (c < 128))
    return row[:S], row[S:], ns, S


def decode_leg(mkv, torch, dev, inp, args, K, V, q, basis, detailed: bool):
    """Compresses the workload once (timed as its own leg), then times decode steps: warmup, an optional
    per-kernel breakdown and unprofiled region (detailed), and the timed region of exactly ``args.steps`` steps
    with HIP events around the score kernel of its first quarter.  Returns (result dict, handles for further
    extras)."""
    w = inp.workload
    bv = 2 if w.dtype == "bf16" else 4
    policy = mkv.mkv_default_policy()
    keep = policy.keeps()
    sb, tb = mkv.mkv_compress_bytes(K, V, inp.cu_seqlens, policy)
    store_buf = torch.empty(sb, dtype=torch.uint8, device=dev)
    scratch = torch.empty(tb, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    store = mkv.mkv_compress(K, V, inp.cu_seqlens, basis, policy, store_buf=store_buf, scratch=scratch)
    torch.cuda.synchronize()
    c_reps = 3
    mkv.mkv_profile_start()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(c_reps):
        store.close()
        store = mkv.mkv_compress(K, V, inp.cu_seqlens, basis, policy, store_buf=store_buf, scratch=scratch)
    e1.record(stream)
    torch.cuda.synchronize()
    c_kern = mkv.mkv_profile_stop()
    compress_ms = e0.elapsed_time(e1) / c_reps
    del scratch
    payload = store.payload_bytes()
    info = store.view()
    S = int(info.segments_per_tensor)
    base = store_buf.data_ptr()
    codes = store_buf[info.codes - base: info.codes - base + 2 * S].cpu().numpy()
    k_rows, v_rows, ns, S = store_bytes(codes, inp.cu_seqlens, w.n_kv_heads, keep, bv)
    k_payload = int((k_rows * ns).sum())
    total_tokens = int(inp.cu_seqlens[-1])
    dense = 2 * total_tokens * w.n_kv_heads * 128 * bv
    n_basis_bytes = w.batch * w.n_kv_heads * 2 * 128 * 128 * 4
    compress_alg_bytes = dense + payload + 9 * 2 * S + n_basis_bytes
    rot_flops = 2.0 * 2 * total_tokens * w.n_kv_heads * 128 * 128
    # segment mix of the stored K and V (share of segments at each kept count)
    mix = {str(keep[c]): float(np.mean(codes.astype(np.int64) == c)) for c in range(len(keep))}

    T = inp.T
    out = torch.empty((w.batch, w.n_q_heads, 128), dtype=torch.float32, device=dev)
    te = np.minimum(T, np.diff(inp.cu_seqlens))
    sel = torch.empty((w.batch, w.n_kv_heads, max(int(te.max()), 1)), dtype=torch.int32, device=dev)
    ws = torch.empty(mkv.mkv_decode_workspace_bytes(store, w.n_q_heads, T), dtype=torch.uint8, device=dev)

    def step():
        mkv.mkv_decode_attn(store, q, T, out=out, sel=sel, ws=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    res = {}
    if detailed:
        # per-kernel breakdown: events around every kernel, which lengthens the step a little
        mkv.mkv_profile_start()
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        kern = mkv.mkv_profile_stop()
        res["kernels_avg_ms"] = {k: v[0] / max(v[1], 1) for k, v in kern.items()}
        # unprofiled region
        t0 = time.perf_counter()
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        res["ms_per_step_unprofiled"] = (time.perf_counter() - t0) * 1e3 / args.steps
    # timed region: events around the score kernel (its roofline) of the first quarter of the steps, nothing else
    # added to the stream.  Each event pair lengthens its step by ~5 us (8 at 1 x 1M; measured with events on one
    # kernel per step, whichever kernel carries them), so events on every launch would charge ~1.5% of the step to
    # the measurement itself; the sampled launches give the kernel's average duration.
    torch.cuda.synchronize()
    roofline_launches = max(1, args.steps // 4)
    mkv.mkv_profile_start(max_launches=roofline_launches, kernels=["score"])
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    score_kern = mkv.mkv_profile_stop()

    sel_np = sel.cpu().numpy()
    n = np.diff(inp.cu_seqlens)
    S_r = (n + 63) // 64
    seg_base = np.concatenate([[0], np.cumsum(S_r)[:-1]])
    v_sel_bytes = 0
    v_segs = 0
    for r in range(w.batch):
        for h in range(w.n_kv_heads):
            j = sel_np[r, h, :te[r]]
            gs = w.n_kv_heads * seg_base[r] + h * S_r[r] + (j >> 6)
            v_sel_bytes += int(v_rows[gs].sum())
            v_segs += int(np.unique(gs).size)
    q_bytes = w.batch * w.n_q_heads * 128 * bv
    out_bytes = w.batch * w.n_q_heads * 128 * 4
    step_alg = k_payload + v_sel_bytes + 9 * (S + v_segs) + q_bytes + out_bytes + n_basis_bytes
    score_ms, score_n = score_kern.get("score", (float("nan"), 0))
    score_avg = score_ms / max(score_n, 1)
    score_alg = k_payload + 9 * S + w.batch * w.n_kv_heads * 128 * 4
    achieved = score_alg / (score_avg * 1e-3) / 1e9
    res.update({
        "ms_per_step": ms,
        "context_tokens_per_s": total_tokens / (ms * 1e-3),
        "score": {"achieved_GBps": achieved, "frac": achieved / HBM_PEAK_GBPS, "alg_bytes_per_launch": score_alg,
                  "avg_launch_ms": score_avg, "timed_launches": score_n},
        "step_alg_bytes": step_alg,
        "step_alg_GBps": step_alg / (ms * 1e-3) / 1e9,
        "step_frac_of_hbm_peak": step_alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
        "store": {"payload_bytes": payload, "dense_kv_bytes": dense, "compression_ratio": dense / payload,
                  "k_payload_bytes": k_payload, "v_selected_bytes": v_sel_bytes, "segment_mix": mix},
        "compress": {"ms": compress_ms, "context_tokens_per_s": total_tokens / (compress_ms * 1e-3),
                     "alg_bytes": compress_alg_bytes, "alg_GBps": compress_alg_bytes / (compress_ms * 1e-3) / 1e9,
                     "alg_frac_of_hbm_peak": compress_alg_bytes / (compress_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                     "rotation_TFLOPs": rot_flops / (compress_ms * 1e-3) / 1e12,
                     "rotation_frac_of_bf16_mfma_peak": rot_flops / (compress_ms * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS,
                     "kernels_avg_ms": {k: v[0] / max(v[1], 1) for k, v in c_kern.items()}},
    })
    handles = {"store": store, "store_buf": store_buf, "out": out, "sel": sel, "step": step, "stream": stream,
               "payload": payload, "dense": dense, "total_tokens": total_tokens, "bv": bv, "policy": policy,
               "T": T}
    return res, handles


def dense_leg(mkv, torch, dev, inp, args, K, V, q, compressed_ms):
    """The uncompressed baseline on the same inputs (bf16 only): the whole call timed, HIP events around its
    attention kernel in the first quarter of the steps."""
    w = inp.workload
    bv = 2
    total_tokens = int(inp.cu_seqlens[-1])
    dense = 2 * total_tokens * w.n_kv_heads * 128 * bv
    dws = torch.empty(mkv.mkv_dense_decode_workspace_bytes(K, V, inp.cu_seqlens, w.n_q_heads), dtype=torch.uint8,
                      device=dev)
    dout = torch.empty((w.batch, w.n_q_heads, 128), dtype=torch.float32, device=dev)

    def dstep():
        mkv.mkv_dense_decode_attn(K, V, inp.cu_seqlens, q, out=dout, ws=dws)

    for _ in range(args.warmup):
        dstep()
    torch.cuda.synchronize()
    # events on the attention kernel of the first quarter of the steps, as for the compressed step
    mkv.mkv_profile_start(max_launches=max(1, args.steps // 4), kernels=["dense_attend"])
    t0 = time.perf_counter()
    for _ in range(args.steps):
        dstep()
    torch.cuda.synchronize()
    dms = (time.perf_counter() - t0) * 1e3 / args.steps
    dk = mkv.mkv_profile_stop()
    d_attend_ms = dk["dense_attend"][0] / max(dk["dense_attend"][1], 1)
    dense_bytes = dense + w.batch * w.n_q_heads * 128 * (bv + 4)
    return {"ms_per_step": dms, "context_tokens_per_s": total_tokens / (dms * 1e-3),
            "alg_bytes": dense_bytes, "attend_kernel_ms": d_attend_ms,
            "attend_kernel_GBps": dense_bytes / (d_attend_ms * 1e-3) / 1e9,
            "attend_kernel_frac_of_hbm_peak": dense_bytes / (d_attend_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
            "attend_kernel_traffic": read_traffic("dense_attend", w.name),
            "compressed_speedup": dms / compressed_ms}


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path (asked for --gpus {args.gpus}); "
              f"run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    w = W.get(args.workload)
    t_gen = time.time()
    inp = W.generate(w, basis="svd", workers=args.workers)
    t_gen = time.time() - t_gen
    # the other workloads the target names (1 x 1M, the ragged mix) and the single-layer Llama shape, measured
    # as extras with the same legs; generated here, before the GPU is touched, with the forked workers
    extra_names = [x for x in args.extras.split(",") if x and x != w.name] if args.extras else []
    extra_inp = {}
    for name in extra_names:
        t1 = time.time()
        extra_inp[name] = (W.generate(W.get(name), basis="svd", workers=args.workers), time.time() - t1)
    # layer-batched extra: the 32 layers of a Llama-3.1-8B-shaped model at 32768 tokens as one store (generated
    # here, before the GPU is touched, like the main inputs)
    lw = W.Workload("llama_32_layers", 32, 32, 8, (32768,) * 32, "bf16", (2048,) * 32, "per_request", 50,
                    "the 32 layers of one 32768-token request, one store")
    linp = W.generate(lw, basis="svd", workers=args.workers) if args.layers else None
    # the oracle's CPU baseline runs before the GPU is touched (its process pool forks this process)
    cpu_base = None if args.no_cpu_baseline else cpu_baseline(inp, args.cpu_seconds, args.workers)

    import torch
    import kv_cache_compression_svd_amd as mkv
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from _helpers import inputs_to_torch

    # The timed loops run Python between kernel launches; a full garbage collection inside one (tens of ms with
    # torch loaded) stalls the launches and would be charged to the GPU.  Collect once here, keep what exists
    # out of later collections, and leave the collector off for the GPU legs (this process is short-lived).
    gc.collect()
    gc.freeze()
    gc.disable()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    K, V, q, basis = inputs_to_torch(inp, dev)
    main_res, H = decode_leg(mkv, torch, dev, inp, args, K, V, q, basis, detailed=True)
    ms = main_res["ms_per_step"]
    store, step, stream = H["store"], H["step"], H["stream"]
    out, sel, T, policy = H["out"], H["sel"], H["T"], H["policy"]
    payload, dense, total_tokens, bv = H["payload"], H["dense"], H["total_tokens"], H["bv"]

    # per-call latency (an extra): events on the stream around each call, back to back and with the 256 MB
    # MALL flushed before every call by reading a 512 MB buffer outside the events (a read leaves clean lines;
    # a fill would leave dirty ones whose write-back would be charged to the next call)
    flush_buf = torch.ones(512 << 20, dtype=torch.uint8, device=dev)

    def per_call(flush):
        evs = []
        for i in range(args.steps):
            if flush:
                flush_buf.view(torch.float32).sum()
            e_a, e_b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e_a.record(stream)
            step()
            e_b.record(stream)
            evs.append((e_a, e_b))
        torch.cuda.synchronize()
        t_ms = np.array([x.elapsed_time(y) for x, y in evs])
        return {"p10_ms": float(np.percentile(t_ms, 10)), "median_ms": float(np.median(t_ms)),
                "p90_ms": float(np.percentile(t_ms, 90)), "calls": int(t_ms.size)}

    call_latency = {"back_to_back": per_call(False), "mall_flushed": per_call(True)}
    del flush_buf

    # uncompressed baseline on the same inputs (an extra): bf16 only
    dense_base = dense_leg(mkv, torch, dev, inp, args, K, V, q, ms) if w.dtype == "bf16" else None

    # Gram matrices for basis refresh on the same inputs (an extra): bf16 only
    gram_res = None
    if w.dtype == "bf16":
        gout = torch.empty((w.batch, w.n_kv_heads, 2, 128, 128), dtype=torch.float32, device=dev)
        for _ in range(2):
            mkv.mkv_gram(K, V, inp.cu_seqlens, out=gout)
        torch.cuda.synchronize()
        mkv.mkv_profile_start(kernels=["gram", "gram_reduce"])
        g_reps = 5
        t0 = time.perf_counter()
        for _ in range(g_reps):
            mkv.mkv_gram(K, V, inp.cu_seqlens, out=gout)
        torch.cuda.synchronize()
        gms = (time.perf_counter() - t0) * 1e3 / g_reps
        gk = mkv.mkv_profile_stop()
        g_kern_ms = gk["gram"][0] / max(gk["gram"][1], 1)
        gram_flops = 2.0 * 2 * total_tokens * w.n_kv_heads * 128 * 128
        gram_res = {"ms": gms, "gram_kernel_ms": g_kern_ms, "alg_bytes": dense,
                    "gram_kernel_GBps": dense / (g_kern_ms * 1e-3) / 1e9,
                    "gram_kernel_frac_of_hbm_peak": dense / (g_kern_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                    "gram_kernel_TFLOPs": gram_flops / (g_kern_ms * 1e-3) / 1e12,
                    "gram_kernel_traffic": read_traffic("gram", args.workload),
                    "reduce_ms": gk["gram_reduce"][0] / max(gk["gram_reduce"][1], 1)}
        del gout

    layer_res = layer_batched(mkv, torch, dev, linp, args) if linp is not None else None

    # incremental append (an extra): a growable store of the same inputs with room for 256 more tokens per
    # request; one append call adds a token to every request (each call re-compresses every open segment)
    append_res = None
    if w.dtype == "bf16":
        n_ctx = np.diff(inp.cu_seqlens)
        gst = mkv.mkv_compress(K, V, inp.cu_seqlens, basis, policy, capacity=n_ctx + 256)
        newK = K[:w.batch * 1].reshape(w.batch, w.n_kv_heads, 128).contiguous()
        newV = V[:w.batch * 1].reshape(w.batch, w.n_kv_heads, 128).contiguous()
        aws = torch.empty(64 * 1024, dtype=torch.uint8, device=dev)
        for _ in range(4):
            mkv.mkv_append(gst, newK, newV, ws=aws)
        torch.cuda.synchronize()
        mkv.mkv_profile_start(kernels=["append"])
        n_app = 64
        t0 = time.perf_counter()
        for _ in range(n_app):
            mkv.mkv_append(gst, newK, newV, ws=aws)
        torch.cuda.synchronize()
        a_ms = (time.perf_counter() - t0) * 1e3 / n_app
        ak = mkv.mkv_profile_stop()
        append_res = {"ms_per_append_call": a_ms, "append_kernel_ms": ak["append"][0] / max(ak["append"][1], 1),
                      "tokens_per_call": w.batch, "streams_recompressed_per_call": 2 * w.batch * w.n_kv_heads,
                      "appended_tokens_per_s": w.batch / (a_ms * 1e-3)}
        del gst

    # paged pool (an extra): the same requests added into a pool of 256 KiB pages, then decoded through a view
    pool_res = None
    if args.pool:
        page = 256 * 1024
        n_pages = int(payload * 1.05) // page + 2 * w.batch * w.n_kv_heads + 64
        grow = 256 if w.dtype == "bf16" else 0   # appendable (bf16): room for 256 more tokens per request
        n_pages += 2 * w.batch * (grow // 64 + 1) * (2 * w.n_kv_heads * 64 * 128 * 2) // page
        pool = mkv.Pool(w.n_kv_heads, mkv.MKV_BF16 if w.dtype == "bf16" else mkv.MKV_FP32, w.batch,
                        int(np.sum((np.diff(inp.cu_seqlens) + grow + 63) // 64)), n_pages, page, policy=policy,
                        appendable=grow > 0)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ids = pool.add(K, V, inp.cu_seqlens, basis, capacity=(np.diff(inp.cu_seqlens) + grow) if grow else None)
        torch.cuda.synchronize()
        add_ms = (time.perf_counter() - t0) * 1e3
        view = pool.view(ids)
        pout = torch.empty_like(out)
        psel = torch.empty_like(sel)
        pws = torch.empty(mkv.mkv_decode_workspace_bytes(view, w.n_q_heads, T), dtype=torch.uint8, device=dev)

        def pstep():
            mkv.mkv_decode_attn(view, q, T, out=pout, sel=psel, ws=pws)

        for _ in range(args.warmup):
            pstep()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            pstep()
        torch.cuda.synchronize()
        p_ms = (time.perf_counter() - t0) * 1e3 / args.steps
        step()
        torch.cuda.synchronize()
        st = pool.stats()
        pool_res = {"page_bytes": page, "pages_used": n_pages - int(st.free_pages), "add_ms": add_ms,
                    "ms_per_step_view": p_ms, "context_tokens_per_s_view": total_tokens / (p_ms * 1e-3),
                    "view_equals_store": bool(torch.equal(pout, out) and torch.equal(psel, sel)),
                    "page_fill": payload / ((n_pages - int(st.free_pages)) * page)}
        if grow:   # one token for every pooled request per call
            newK = K[:w.batch].reshape(w.batch, w.n_kv_heads, 128).contiguous()
            newV = V[:w.batch].reshape(w.batch, w.n_kv_heads, 128).contiguous()
            pws = torch.empty(64 * 1024, dtype=torch.uint8, device=dev)
            for _ in range(4):
                pool.append(ids, newK, newV, ws=pws)
            torch.cuda.synchronize()
            n_app = 64
            t0 = time.perf_counter()
            for _ in range(n_app):
                pool.append(ids, newK, newV, ws=pws)
            torch.cuda.synchronize()
            pool_res["ms_per_append_call"] = (time.perf_counter() - t0) * 1e3 / n_app
        del view, pool

    # the other workloads: their own inputs, compress and decode legs (and the uncompressed baseline)
    del K, V, q, basis, store, H, step, out, sel
    torch.cuda.empty_cache()
    extras = {}
    for name in extra_names:
        einp, gen_s = extra_inp.pop(name)
        eK, eV, eq, eb = inputs_to_torch(einp, dev)
        r, eh = decode_leg(mkv, torch, dev, einp, args, eK, eV, eq, eb, detailed=True)
        ew = einp.workload
        r["config"] = {"batch": ew.batch, "context": list(ew.ctx) if len(set(ew.ctx)) > 1 or ew.batch == 1 else
                       f"{ew.batch} x {ew.ctx[0]}", "q_heads": ew.n_q_heads, "kv_heads": ew.n_kv_heads,
                       "T": int(ew.T[0]) if len(set(ew.T)) == 1 else list(ew.T), "dtype": ew.dtype}
        r["input_generation_s"] = gen_s
        if ew.dtype == "bf16":
            r["dense_baseline"] = dense_leg(mkv, torch, dev, einp, args, eK, eV, eq, r["ms_per_step"])
        extras[name] = r
        del eK, eV, eq, eb, eh, einp
        torch.cuda.empty_cache()

    traffic = read_traffic("score", args.workload)
    result = {
        "metric": METRIC,
        "value": total_tokens / (ms * 1e-3),
        "unit": "context tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "fp32",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "context": list(w.ctx) if w.batch <= 4 else
                   f"{w.batch} x {w.ctx[0]}" if len(set(w.ctx)) == 1 else list(w.ctx),
                   "q_heads": w.n_q_heads, "kv_heads": w.n_kv_heads, "head_dim": 128,
                   "T": int(w.T[0]) if len(set(w.T)) == 1 else list(w.T), "seg_len": 64,
                   "keep": list(policy.keeps()), "energy_frac": 0.9, "accumulate": "fp32",
                   "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "hbm", "kernel": "score", "achieved": main_res["score"]["achieved_GBps"],
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": main_res["score"]["frac"],
                     "traffic": traffic, "alg_bytes_per_launch": main_res["score"]["alg_bytes_per_launch"],
                     "avg_launch_ms": main_res["score"]["avg_launch_ms"],
                     "timed_launches": main_res["score"]["timed_launches"]},
        "step_alg_bytes": main_res["step_alg_bytes"],
        "step_alg_GBps": main_res["step_alg_GBps"],
        "step_frac_of_hbm_peak": main_res["step_frac_of_hbm_peak"],
        "ms_per_step_unprofiled": main_res["ms_per_step_unprofiled"],
        "call_latency": call_latency,
        "kernels_avg_ms": main_res["kernels_avg_ms"],
        "store": main_res["store"],
        "compress": main_res["compress"],
        "dense_baseline": dense_base,
        "gram": gram_res,
        "layer_batched": layer_res,
        "append": append_res,
        "pool": pool_res,
        "workloads": extras,
        "input_generation_s": t_gen,
    }
    if cpu_base is not None:
        result["cpu_baseline"] = cpu_base
    print(json.dumps(result), flush=True)


def layer_batched(mkv, torch, dev, linp, args):
    """All layers of one request decoded by one call (the layers are the store's requests) against one call
    for a single layer: the batched call amortises launches and fills the GPU."""
    from _helpers import inputs_to_torch
    lw = linp.workload
    n = lw.ctx[0]
    K, V, q, basis = inputs_to_torch(linp, dev)
    store = mkv.mkv_compress(K, V, linp.cu_seqlens, basis)
    one = mkv.mkv_compress(K[:n].contiguous(), V[:n].contiguous(), linp.cu_seqlens[:2], basis[:1].contiguous())
    q1 = q[:1].contiguous()
    del K, V

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / args.steps

    out = torch.empty((lw.batch, lw.n_q_heads, 128), dtype=torch.float32, device=dev)
    ws = torch.empty(mkv.mkv_decode_workspace_bytes(store, lw.n_q_heads, linp.T), dtype=torch.uint8, device=dev)
    out1 = torch.empty((1, lw.n_q_heads, 128), dtype=torch.float32, device=dev)
    ws1 = torch.empty(mkv.mkv_decode_workspace_bytes(one, lw.n_q_heads, linp.T[:1]), dtype=torch.uint8, device=dev)
    ms_all = timed(lambda: mkv.mkv_decode_attn(store, q, linp.T, out=out, ws=ws, return_sel=False))
    ms_one = timed(lambda: mkv.mkv_decode_attn(one, q1, linp.T[:1], out=out1, ws=ws1, return_sel=False))
    return {"layers": lw.batch, "context": n, "T": int(linp.T[0]), "ms_one_layer_one_call": ms_one,
            "ms_all_layers_one_call": ms_all, "ms_per_layer_batched": ms_all / lw.batch,
            "speedup_vs_one_call_per_layer": lw.batch * ms_one / ms_all,
            "context_tokens_per_s_batched": lw.batch * n / (ms_all * 1e-3),
            "context_tokens_per_s_one_layer": n / (ms_one * 1e-3)}


def _oracle_unit_rate(inp, unit, seconds: float, blas_threads=None):
    """(context tokens of the unit, decode repetitions, seconds) of the oracle's decode step on one (request,
    KV head) unit, repeated for about ``seconds``; its store is built by the oracle first (untimed)."""
    import oracle
    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=blas_threads):
        streams = oracle.compress_all(inp, units=[unit])
        reps, t = 0, 0.0
        while t < seconds or reps < 1:
            t0 = time.perf_counter()
            oracle.decode_all(inp, streams, units=[unit])
            t += time.perf_counter() - t0
            reps += 1
    r = unit[0]
    return int(inp.cu_seqlens[r + 1] - inp.cu_seqlens[r]), reps, t


_POOL_INP = None


def _pool_worker(args):
    unit, seconds = args
    return _oracle_unit_rate(_POOL_INP, unit, seconds, blas_threads=1)


def cpu_baseline(inp, seconds: float, procs: int):
    """The float64 oracle's decode step timed on the host two ways: (i) one process, BLAS threads = all cores,
    on the (request 0, KV head 0) unit; (ii) a process pool (one BLAS thread each) over ``procs`` independent
    (request, KV head) units, all running at once.  Each unit's store is built by the oracle first, untimed.
    Context tokens/s of a layer = (context-token-heads decoded per second) / n_kv_heads; the reported value is
    the faster of the two."""
    import multiprocessing as mp
    from threadpoolctl import threadpool_info
    global _POOL_INP
    w = inp.workload
    n0, reps, t = _oracle_unit_rate(inp, (0, 0), seconds)
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    single = n0 * reps / (w.n_kv_heads * t)
    units = [(r, h) for r in range(w.batch) for h in range(w.n_kv_heads)][:max(1, procs)]
    _POOL_INP = inp
    with mp.get_context("fork").Pool(len(units)) as pool:
        got = pool.map(_pool_worker, [(u, seconds) for u in units])
    _POOL_INP = None
    pooled = sum(n * k / tt for n, k, tt in got) / w.n_kv_heads
    best = max(single, pooled)
    return {"value": best, "unit": "context tokens/s", "cores": len(units) if pooled >= single else threads,
            "kind": "oracle", "cpu_model": cpu_model(), "host_cpu_count": os.cpu_count(),
            "single_process": {"value": single, "blas_threads": threads, "reps": reps, "seconds": t},
            "process_pool": {"value": pooled, "processes": len(units), "blas_threads_each": 1,
                             "units": [list(u) for u in units]},
            "sample": f"float64 numpy oracle decode: (i) request 0 / KV head 0 ({n0} tokens, T={int(inp.T[0])}) "
                      f"repeated {reps}x in {t:.1f}s with {threads} BLAS threads; (ii) {len(units)} (request, KV "
                      f"head) units at once in a process pool, one BLAS thread each, ~{seconds:.0f}s each; stores "
                      f"compressed by the oracle beforehand, untimed; tokens/s = context-token-heads per second / "
                      f"{w.n_kv_heads} KV heads; host cpu_count {os.cpu_count()}"}


if __name__ == "__main__":
    main()
