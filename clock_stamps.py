#!/usr/bin/env python3
"""Per-workgroup clocks of the decode-attention kernel (measurement tool).

Loads the measurement build kv_cache_compression_mla_amd/libmla_stamps.so (the
library with per-workgroup stamps in the attention kernel: the shader-clock
counter s_memtime, which counts shader cycles, and the 100 MHz real-time
counter s_memrealtime, read at each workgroup's start and end), runs the
attention call of one workload back to back, and reports for the last call
the shader cycles of every workgroup, its real time and the clock it ran at
(cycles over real time), for two caches of the same geometry:

  contiguous    the workload's own cache (64 sequences of 8193 distinct rows
                at the headline size): every row streams from HBM
  paged         the same rows copied into a pool of 64-row pages, each
                sequence with its own pages: streams from HBM, paged addressing
  paged_shared  a pool holding one sequence's rows, every sequence's block
                table listing the same pages: the same attended rows, chunk
                plan and addressing, but only 9.4 MB of distinct rows at the
                headline size, which the caches serve after the first call

The kernel does the same work on the two paged caches; comparing them
separates the cycles the kernel needs from the clock the chip runs it at.

With --phases W [W ...] it instead runs each named workload on its own cache
(contiguous or paged, as the workload defines it) and reports, per phase of
the kernel, the median shader cycles of the workgroups from the phase stamps
wave 0 takes: the chunk plan, the prologue (query block, first copies, first
tile's scores and weights), the steady loop, the general loop (last
iterations), the last value step with the fallback check, the (m, l) write,
and the epilogue (output or partials).

Usage: python3 clock_stamps.py [--workload v3_b64_ctx8k] [--calls 200]
       python3 clock_stamps.py --phases v3_b64_ctx8k v3_b8_ctx32k
Prints one JSON line per cache (or workload) and a markdown table.
"""
import argparse
import ctypes
import json
import os
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--workload", default="v3_b64_ctx8k")
    ap.add_argument("--calls", type=int, default=200)
    ap.add_argument("--phases", nargs="+", metavar="WORKLOAD")
    args = ap.parse_args()

    import numpy as np
    import torch
    from kv_cache_compression_mla_amd import build as bld
    from kv_cache_compression_mla_amd import inputs as gen
    from kv_cache_compression_mla_amd import mla
    from kv_cache_compression_mla_amd.step import DeviceStep

    if not os.path.exists(bld.LIB_STAMPS):
        raise SystemExit(f"{bld.LIB_STAMPS} is missing: build it first (__graft_entry__.build())")
    assert torch.cuda.is_available(), "clock_stamps.py needs a GPU"
    L = ctypes.CDLL(bld.LIB_STAMPS)
    attn = L.mla_decode_attn
    attn.restype, attn.argtypes = mla._SIGS["mla_decode_attn"]
    stamps = L.mla_clock_stamps
    stamps.restype, stamps.argtypes = ctypes.c_int, [ctypes.c_void_p, ctypes.c_int]

    if args.phases:
        phases(L, attn, args.phases, args.calls)
        return
    cfg = gen.CONFIGS[args.workload]
    assert not cfg.paged and not cfg.topk, "a contiguous dense workload"
    inp = gen.make_inputs(cfg)
    st = DeviceStep(inp)
    st.run()                              # the query, from the product library
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    # the balanced plan launches one workgroup per compute unit
    grid = max(torch.cuda.get_device_properties(0).multi_processor_count, cfg.B)

    # paged copies: every sequence on its own pages, and one sequence's rows
    # on pages that every sequence's table lists
    bs = 64
    L0 = int(inp.seq_lens[0])
    assert (inp.seq_lens == L0).all(), "equal lengths"
    npages = (L0 + bs - 1) // bs
    pool_own = torch.zeros(cfg.B * npages * bs, cfg.D, dtype=st.cache.dtype, device="cuda")
    for b in range(cfg.B):
        pool_own[b * npages * bs:b * npages * bs + L0] = st.cache[b, :L0]
    pool_own = pool_own.view(cfg.B * npages, bs, cfg.D)
    table_own = torch.arange(cfg.B * npages, dtype=torch.int32, device="cuda").view(cfg.B, npages).contiguous()
    pool_shared = pool_own[:npages].contiguous()
    table_shared = torch.arange(npages, dtype=torch.int32, device="cuda").repeat(cfg.B, 1).contiguous()
    caches = (("contiguous", st.cdesc), ("paged", mla.make_cache(pool_own, table_own)),
              ("paged_shared", mla.make_cache(pool_shared, table_shared)))

    results = []
    for name, cdesc in caches:
        def call():
            rc = attn(ctypes.byref(st.dims), cfg.B, st.q.data_ptr(), ctypes.byref(cdesc), st.seq_lens.data_ptr(),
                      st.max_seq_len, 0, st.o_lat.data_ptr(), st.lse.data_ptr(), st.ws.data_ptr(), st.ws.numel(),
                      stream.cuda_stream)
            if rc != 0:
                raise RuntimeError(mla.lib().mla_status_str(rc).decode())
        for _ in range(20):
            call()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.calls):
            call()
        e1.record(stream)
        torch.cuda.synchronize()
        per_call_us = e0.elapsed_time(e1) / args.calls * 1e3
        buf = np.zeros((grid, 4), dtype=np.uint64)
        rc = stamps(buf.ctypes.data, grid)
        if rc != 0:
            raise RuntimeError(f"mla_clock_stamps failed ({rc})")
        s = buf.astype(np.float64)
        cyc = s[:, 1] - s[:, 0]
        us = (s[:, 3] - s[:, 2]) / 100.0
        ghz = cyc / us / 1e3
        span_us = (s[:, 3].max() - s[:, 2].min()) / 100.0
        tiles = (L0 + 31) // 32 * cfg.B / grid
        res = {"cache": name, "workload": cfg.name, "calls": args.calls, "workgroups": grid,
               "call_us": round(per_call_us, 1), "last_call_span_us": round(span_us, 1),
               "cycles_median": int(np.median(cyc)), "cycles_max": int(cyc.max()),
               "cycles_per_tile_median": int(np.median(cyc) / tiles),
               "wg_time_us_median": round(float(np.median(us)), 1), "wg_time_us_max": round(float(us.max()), 1),
               "clock_ghz_median": round(float(np.median(ghz)), 3), "clock_ghz_min": round(float(ghz.min()), 3),
               "clock_ghz_max": round(float(ghz.max()), 3)}
        results.append(res)
        print(json.dumps(res), flush=True)
    print("\n| cache | call (us) | cycles per workgroup (median) | cycles per 32-row tile | "
          "workgroup time (us, median / max) | clock GHz (median, min..max) |")
    print("|---|---:|---:|---:|---|---|")
    for r in results:
        print(f"| {r['cache']} | {r['call_us']} | {r['cycles_median']:,} | {r['cycles_per_tile_median']:,} | "
              f"{r['wg_time_us_median']} / {r['wg_time_us_max']} | {r['clock_ghz_median']} "
              f"({r['clock_ghz_min']}..{r['clock_ghz_max']}) |")


PHASES = ["plan", "prologue", "steady loop", "general loop", "last value step", "(m, l) write", "epilogue"]


def phases(L, attn, workloads, calls):
    import numpy as np
    import torch
    from kv_cache_compression_mla_amd import inputs as gen
    from kv_cache_compression_mla_amd import mla
    from kv_cache_compression_mla_amd.step import DeviceStep

    ph = L.mla_phase_stamps
    ph.restype, ph.argtypes = ctypes.c_int, [ctypes.c_void_p, ctypes.c_int]
    reset = L.mla_clock_stamps_reset
    reset.restype, reset.argtypes = ctypes.c_int, []
    assert calls >= 2
    rows = []
    for name in workloads:
        cfg = gen.CONFIGS[name]
        assert not cfg.topk, "a dense workload"
        st = DeviceStep(gen.make_inputs(cfg))
        st.run()
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream()
        for _ in range(calls):
            rc = attn(ctypes.byref(st.dims), cfg.B, st.q.data_ptr(), ctypes.byref(st.cdesc), st.seq_lens.data_ptr(),
                      st.max_seq_len, 0, st.o_lat.data_ptr(), st.lse.data_ptr(), st.ws.data_ptr(), st.ws.numel(),
                      stream.cuda_stream)
            if rc != 0:
                raise RuntimeError(mla.lib().mla_status_str(rc).decode())
            if _ == calls - 2:
                # before the last call: only its workgroups with a chunk stamp
                torch.cuda.synchronize()
                if reset() != 0:
                    raise RuntimeError("mla_clock_stamps_reset failed")
        torch.cuda.synchronize()
        grid = max(torch.cuda.get_device_properties(0).multi_processor_count, cfg.B)
        buf = np.zeros((grid, 8), dtype=np.uint64)
        if ph(buf.ctypes.data, grid) != 0:
            raise RuntimeError("mla_phase_stamps failed")
        s = buf[buf[:, 7] > buf[:, 0]].astype(np.float64)
        total = len(s)
        d = np.diff(s, axis=1)
        res = {"workload": name, "workgroups": total, "calls": calls,
               "cycles_median": int(np.median(s[:, 7] - s[:, 0]))}
        res.update({k: int(np.median(d[:, i])) for i, k in enumerate(PHASES)})
        rows.append(res)
        print(json.dumps(res), flush=True)
    print("\n| workload | " + " | ".join(PHASES) + " | workgroup |")
    print("|---|" + "---:|" * (len(PHASES) + 1))
    for r in rows:
        print(f"| {r['workload']} | " + " | ".join(f"{r[k]:,}" for k in PHASES) + f" | {r['cycles_median']:,} |")


if __name__ == "__main__":
    main()
