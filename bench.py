#!/usr/bin/env python3
"""MLA decode benchmark on one MI355X.

One step = the whole decode hot path over one batch: compress + RoPE + append
of the new tokens, absorbed query, latent-space attention against the cache
(with the cross-split combine), and the output projections. Inputs are seeded
synthetic tensors of the DeepSeek-V3 geometry, resident in HBM before timing.

Headline: decode-attention TFLOP/s (algorithmic FLOPs 2*H*(D + d_c) per
attended row) and latent-cache GB/s (1152 B per attended row) of the
mla_decode_attn call. The call's kernels stamp HIP events themselves
(mla_time_next_attn: hipExtLaunchKernel's start and stop events on the stream
the library launches on), so the timed steps carry no marker commands: attn_ms
runs from the attention kernel's start to the end of the merge of the chunks
(combine_chunks), attn_kernel_ms is the attention kernel alone. The roofline
object prices that kernel, the dominant one, against MI355X's published HBM
bandwidth (8 TB/s) with its algorithmic bytes (cache rows and q, and o_lat
when no merge runs); the "call" object prices the whole call (cache, q,
o_lat, lse). ms_per_step is the whole step (wall clock over the K timed
steps) and calls_ms the mean time of each of the four calls from a separate
untimed pass with marker events between them. The CPU baseline times the
float64 oracle on a bounded sample of the same workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                       [--precomposed]
--precomposed runs the query and output sides with the composed weights
W_QK = W_UK^T W_UQ and W_OV = W_O blockdiag(W_UV), formed before timing.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0       # MI355X dense bf16 MFMA, published
ATTN_SRC = os.path.join(ROOT, "kv_cache_compression_mla_amd", "csrc", "attn_mfma.hip")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def attn_work(cfg, seq_lens):
    """Algorithmic bytes and FLOPs of one attention call (seq_lens: rows
    attended per sequence; the entry counts for sparse attention): rows,
    cache bytes, q bytes, o_lat + lse bytes, FLOPs."""
    rows = int(seq_lens.sum())
    row_bytes = cfg.D * 2
    cache_bytes = rows * row_bytes
    q_bytes = cfg.B * cfg.H * (cfg.D + cfg.d_R) * 2     # [q_lat ; q_R ; low term of q_R]
    out_bytes = cfg.B * cfg.H * cfg.d_c * 4 + cfg.B * cfg.H * 4
    flops = rows * 2 * cfg.H * (cfg.D + cfg.d_c)
    return rows, cache_bytes, q_bytes, out_bytes, flops


def traffic_from_profile(workload):
    """HBM bytes per launch of the attention kernel and per attention call
    (kernel + merge) from committed rocprofv3 counter runs, if they were taken
    on the current kernel source; else (None, None)."""
    path = os.path.join(ROOT, "profiles", f"attn_hbm_traffic_{workload}.json")
    if not os.path.exists(path):
        return None, None
    try:
        with open(path) as f:
            prof = json.load(f)
        with open(ATTN_SRC, "rb") as f:
            src_hash = hashlib.sha256(f.read()).hexdigest()
        if prof.get("attn_source_sha256") != src_hash:
            return None, None
        k = prof["kernels"]["attn"]
        return round(k["fetch_bytes"] + k["write_bytes"]), prof.get("bytes_per_call")
    except Exception:
        return None, None


def cpu_baseline(inp, budget_s, topk=None):
    """Time the float64 oracle (unabsorbed: per-head K and V rebuilt from every
    attended latent) on whole sequences of the workload until the budget is
    used. topk: (indices, counts) for sparse attention."""
    import numpy as np
    from kv_cache_compression_mla_amd import inputs as gen
    from oracle import mla_oracle as om
    cfg = inp.cfg
    cores = len(os.sched_getaffinity(0))
    W = {k: (None if v is None else gen.to_f64(v, cfg.dtype)) for k, v in inp.weights.items()}
    done_rows, t_used, nseq = 0, 0.0, 0
    for b in range(cfg.B):
        h = gen.to_f64(inp.h_t[b], cfg.dtype)
        prior = gen.to_f64(inp.rows(b, int(inp.ctx[b])), cfg.dtype)
        idx = None if topk is None else topk[0][b, :int(topk[1][b])]
        t0 = time.perf_counter()
        om.decode_step(h, prior, W, int(inp.ctx[b]), cfg.theta, cfg.scale, cfg.dtype, idx=idx)
        t_used += time.perf_counter() - t0
        done_rows += int(inp.seq_lens[b]) if topk is None else int(topk[1][b])
        nseq += 1
        if t_used >= budget_s:
            break
    flops = done_rows * 2 * cfg.H * (cfg.D + cfg.d_c)
    return {"value": flops / t_used / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"{nseq} of {cfg.B} sequences ({done_rows} attended rows, all {cfg.H} heads), "
                      f"float64 numpy unabsorbed step, {t_used:.1f} s; value counts the same "
                      f"algorithmic attention FLOPs as the GPU line"}


def cpu_fair(inp, budget_s, topk=None):
    """A fair CPU line beside the oracle: the absorbed decode attention as a
    CPU would run it, in float32 numpy (BLAS on the host cores) against the
    same latent rows. Per sequence: scores = q_lat.rows^T over 576 columns for
    all heads at once, softmax over the rows, o_lat = P.rows[:, :512]. The
    query is a seeded draw of the absorbed query's shape; rows are upcast
    before timing. Counts the same algorithmic FLOPs as the GPU line."""
    import numpy as np
    from kv_cache_compression_mla_amd import inputs as gen
    cfg = inp.cfg
    cores = len(os.sched_getaffinity(0))
    q = gen.to_f64(gen.make_query(cfg), cfg.dtype).astype(np.float32)
    done_rows, t_used, nseq = 0, 0.0, 0
    for b in range(cfg.B):
        L = int(inp.ctx[b])
        rows = gen.to_f64(inp.rows(b, L), cfg.dtype).astype(np.float32)
        rows = np.concatenate([rows, rows[-1:]], axis=0) if L else rows   # the appended row's slot
        if topk is not None:
            rows = rows[np.asarray(topk[0][b, :int(topk[1][b])], dtype=np.int64)]
        t0 = time.perf_counter()
        s = (q[b] @ rows.T) * np.float32(cfg.scale)                       # [H][L]
        s -= s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p /= p.sum(axis=1, keepdims=True)
        o = p @ rows[:, :cfg.d_c]                                          # [H][d_c]
        t_used += time.perf_counter() - t0
        assert np.isfinite(o).all()
        done_rows += rows.shape[0]
        nseq += 1
        if t_used >= budget_s:
            break
    flops = done_rows * 2 * cfg.H * (cfg.D + cfg.d_c)
    return {"value": flops / t_used / 1e12, "unit": "TFLOP/s", "cores": cores,
            "kind": "absorbed float32 numpy (not the oracle)",
            "sample": f"{nseq} of {cfg.B} sequences ({done_rows} attended rows, all {cfg.H} heads), "
                      f"{t_used:.2f} s of timed attention"}


def prefill_work(cfg, seq_lens, T, rows_stored):
    """Algorithmic FLOPs of causal prefill of the newest T tokens, per algorithm.
    Attended rows: token t of a sequence of L rows sees L - T + t + 1 of them.
    Materialised: expanding every stored row, 2 d_c H (d_h + d_v) per row, then
    2 H (d_h + d_R + d_v) per attended row. Absorbed: W_UK^T per token
    (2 H d_h d_c), 2 H (2 d_c + d_R) per attended row, W_UV per token (2 H d_c d_v)."""
    att = 0
    for L in seq_lens:
        L = int(L)
        att += sum(max(0, L - T + t + 1) for t in range(T))
    H = cfg.H
    mat = 2 * rows_stored * cfg.d_c * H * (cfg.d_h + cfg.d_v) + 2 * H * (cfg.d_h + cfg.d_R + cfg.d_v) * att
    ntok = len(seq_lens) * T
    absb = (2 * ntok * H * cfg.d_h * cfg.d_c + 2 * H * (2 * cfg.d_c + cfg.d_R) * att
            + 2 * ntok * H * cfg.d_c * cfg.d_v)
    return att, mat, absb


def prefill_sweep(Ts, steps, warmup):
    """Causal prefill of the newest T tokens of 4 sequences of 4096 cached rows:
    the materialised form (expand every row's per-head keys and values, then
    per-head causal attention) against the absorbed form (latent attention,
    one entry per token), same inputs and outputs, timed with HIP events on
    the stream the library launches on."""
    import numpy as np
    import torch
    from kv_cache_compression_mla_amd import inputs as gen
    from kv_cache_compression_mla_amd import mla
    from kv_cache_compression_mla_amd.step import DevicePrefill
    cfg = gen.CONFIGS["v3_b4_ctx4k_prefill"]
    inp = gen.make_inputs(cfg)
    stream = torch.cuda.current_stream()
    for T in Ts:
        pf = DevicePrefill(inp, T)
        rows_stored = cfg.B * inp.cache.shape[1]
        att, f_mat, f_abs = prefill_work(cfg, pf.seq_lens_host, T, rows_stored)
        res = {"workload": cfg.name, "T": T, "tokens": cfg.B * T, "rows_attended": att}
        for name, algo, flops in (("materialised", mla.PREFILL_MATERIALIZED, f_mat),
                                  ("absorbed", mla.PREFILL_ABSORBED, f_abs)):
            for _ in range(warmup):
                pf.run(algo)
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
            torch.cuda.synchronize()
            for a, b in ev:
                a.record(stream)
                pf.run(algo)
                b.record(stream)
            torch.cuda.synchronize()
            ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
            res[name] = {"ms": round(ms, 4), "GFLOP": round(flops / 1e9, 2),
                         "TFLOP/s": round(flops / (ms * 1e-3) / 1e12, 1)}
        res["faster"] = min(("materialised", "absorbed"), key=lambda k: res[k]["ms"])
        pick = mla.prefill_choose(pf.dims, cfg.B, T, pf.max_seq_len, pf.cdesc)
        res["auto_picks"] = {mla.PREFILL_MATERIALIZED: "materialised", mla.PREFILL_ABSORBED: "absorbed"}.get(pick)
        print(json.dumps(res), flush=True)
        del pf
        torch.cuda.empty_cache()


class DeviceEvents:
    """HIP events for timing the attention call on the library's stream,
    created with hipEventReleaseToDevice: recording one performs a
    device-scope release instead of the default system-scope one, which the
    HIP runtime documents as the way to time the commands between events more
    precisely (the default event writes back and invalidates caches for the
    host, and that costs the kernels after it). The events come from the HIP
    runtime torch itself loaded, so they share its streams."""
    RELEASE_TO_DEVICE = 0x40000000

    def __init__(self, torch):
        import ctypes
        self.ct = ctypes
        path = os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so")
        if not os.path.exists(path):
            path = "/opt/rocm/lib/libamdhip64.so"
        self.hip = ctypes.CDLL(path)
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.events = []

    def create(self):
        e = self.ct.c_void_p()
        rc = self.hip.hipEventCreateWithFlags(self.ct.byref(e), self.RELEASE_TO_DEVICE)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")
        self.events.append(e)
        return e

    def record(self, e, stream):
        rc = self.hip.hipEventRecord(e, self.ct.c_void_p(stream.cuda_stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def elapsed_ms(self, a, b):
        ms = self.ct.c_float()
        rc = self.hip.hipEventElapsedTime(self.ct.byref(ms), a, b)
        if rc != 0:
            # take the error off the thread, or the next HIP call (torch's
            # included) reports it as its own
            self.hip.hipGetLastError()
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def close(self):
        for e in self.events:
            self.hip.hipEventDestroy(e)
        self.events = []


def measured_copy_gbps(torch, nbytes=1 << 30, reps=10):
    """Device-to-device copy rate of this GPU (bytes read + written per
    second), the practical counterpart of the published HBM peak."""
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    gbps = 2 * nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return gbps


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="v3_b64_ctx8k")
    ap.add_argument("--num-splits", type=int, default=0)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--prefill-sweep", default="",
                    help="comma-separated token counts T: time causal prefill of the newest T tokens of "
                         "v3_b4_ctx4k_prefill, materialised against absorbed (one JSON line per T)")
    ap.add_argument("--precomposed", action="store_true",
                    help="query and output sides with composed weights W_QK, W_OV (formed before timing)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the decode path is "
              "single-GPU in this build. Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from kv_cache_compression_mla_amd import inputs as gen
    from kv_cache_compression_mla_amd import mla
    from kv_cache_compression_mla_amd.step import DeviceStep

    if not os.path.exists(mla.library_path()):
        import __graft_entry__
        __graft_entry__.build()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.prefill_sweep:
        prefill_sweep([int(x) for x in args.prefill_sweep.split(",")], args.steps, args.warmup)
        return
    cfg = gen.CONFIGS[args.workload]
    t0 = time.perf_counter()
    inp = gen.make_inputs(cfg)
    log(f"inputs for {cfg.name} generated in {time.perf_counter() - t0:.1f} s")
    st = DeviceStep(inp, num_splits=args.num_splits, precomposed=args.precomposed)
    attended = st.topk_counts_host if cfg.topk else inp.seq_lens
    rows, cache_bytes, q_bytes, out_bytes, attn_flops = attn_work(cfg, attended)
    attn_bytes = cache_bytes + q_bytes + out_bytes
    splits = st.splits
    # a sequence cut into chunks is merged by a second kernel (combine_chunks),
    # which writes o_lat; otherwise the attention kernel writes it
    merged = splits > 1
    kernel_bytes = cache_bytes + q_bytes + (0 if merged else out_bytes)
    log(f"B={cfg.B} rows={rows} splits={splits} kernel={mla.decode_kernel(st.dims)}")

    stream = torch.cuda.current_stream()
    # timed region: K whole steps. The attention call of each step stamps three
    # events from its own kernel launches (mla_time_next_attn: the attention
    # kernel's start and end, and the end of the merge), so no marker command
    # enters the stream and the step runs as it would untimed.
    dev_ev = DeviceEvents(torch)
    ev = [(dev_ev.create(), dev_ev.create(), dev_ev.create()) for _ in range(args.steps)]
    for _ in range(args.warmup):
        st.run()
    torch.cuda.synchronize()

    t_start = time.perf_counter()
    for k in range(args.steps):
        st.compress_append()
        st.absorb_q()
        mla.mla_time_next_attn(ev[k][0].value, ev[k][1].value, ev[k][2].value)
        st.decode_attn()
        st.out_proj()
    torch.cuda.synchronize()
    t_total = time.perf_counter() - t_start
    attn_times = [dev_ev.elapsed_ms(a, c) for a, b, c in ev]
    kernel_times = [dev_ev.elapsed_ms(a, b) for a, b, c in ev]
    attn_ms = float(np.mean(attn_times))
    kernel_ms = float(np.mean(kernel_times))
    ms_per_step = t_total * 1e3 / args.steps

    # per-call breakdown, after the timed region: events between all four calls
    calls = ("compress_append", "absorb_q", "decode_attn", "out_proj")
    nb = min(args.steps, 10)
    evc = [[dev_ev.create() for _ in range(len(calls) + 1)] for _ in range(nb)]
    for e in evc:
        dev_ev.record(e[0], stream)
        st.compress_append()
        dev_ev.record(e[1], stream)
        st.absorb_q()
        dev_ev.record(e[2], stream)
        st.decode_attn()
        dev_ev.record(e[3], stream)
        st.out_proj()
        dev_ev.record(e[4], stream)
    torch.cuda.synchronize()
    calls_ms = {c: round(float(np.mean([dev_ev.elapsed_ms(e[i], e[i + 1]) for e in evc])), 5)
                for i, c in enumerate(calls)}

    copy_gbps = measured_copy_gbps(torch)
    tflops = attn_flops / (attn_ms * 1e-3) / 1e12
    cache_gbps = cache_bytes / (attn_ms * 1e-3) / 1e9
    call_gbps = attn_bytes / (attn_ms * 1e-3) / 1e9
    kernel_gbps = kernel_bytes / (kernel_ms * 1e-3) / 1e9
    kernel_traffic, call_traffic = traffic_from_profile(cfg.name)
    result = {
        "metric": "MLA decode-attn TFLOP/s + cache GB/s (% roofline), H=128 d_c=512+64, bs64 ctx8K",
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "batch": cfg.B, "ctx": int(inp.ctx.max()),
                   "rows_attended": rows, "heads": cfg.H, "d_c": cfg.d_c, "d_R": cfg.d_R,
                   "paged": cfg.paged, "num_splits": splits, "topk": cfg.topk,
                   "precomposed": bool(args.precomposed)},
        "attn_ms": round(attn_ms, 5),
        "attn_ms_median": round(float(np.median(attn_times)), 5),
        "attn_kernel_ms": round(kernel_ms, 5),
        "calls_ms": calls_ms,
        "cache_GBps": round(cache_gbps, 1),
        "pct_hbm_roofline": round(100 * call_gbps / HBM_PEAK_GBPS, 2),
        "roofline": {"bound": "hbm", "achieved": round(kernel_gbps, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(kernel_gbps / HBM_PEAK_GBPS, 4),
                     "traffic": kernel_traffic,
                     "kernel": "attn_mfma_kernel (algorithmic bytes: cache rows + q"
                               + (")" if merged else " + o_lat + lse)"),
                     "bytes": kernel_bytes,
                     "measured_copy_GBps": round(copy_gbps, 1),
                     "frac_of_copy": round(kernel_gbps / copy_gbps, 4),
                     "mfma_frac": round(attn_flops / (kernel_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)},
        "call": {"what": "mla_decode_attn, attention kernel start to "
                         + ("combine_chunks end" if merged else "its end"),
                 "ms": round(attn_ms, 5), "bytes": attn_bytes, "achieved_GBps": round(call_gbps, 1),
                 "frac": round(call_gbps / HBM_PEAK_GBPS, 4), "traffic": call_traffic},
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle ...")
        tk = (st.topk_idx_host, st.topk_counts_host) if cfg.topk else None
        result["cpu_baseline"] = cpu_baseline(inp, args.cpu_seconds, tk)
        log("timing the absorbed float32 CPU attention ...")
        result["cpu_fair"] = cpu_fair(inp, min(5.0, args.cpu_seconds), tk)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
