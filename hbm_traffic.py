"""HBM traffic of the decode-attention call, from rocprofv3 counters.

Two steps, each a plain command:

  run        (on the GPU, under rocprofv3 --pmc FETCH_SIZE, then again under
             --pmc WRITE_SIZE): builds one workload's inputs, makes `calls`
             mla_decode_attn calls, then runs kernels of known traffic on a
             256 MiB float32 buffer: an elementwise copy (x * 1 into another
             buffer: reads and writes 256 MiB, 16-byte vector accesses), a
             fill (writes 256 MiB), a sum (reads 256 MiB) and a runtime
             device-to-device copy (blit kernel);
  summarize  (anywhere): reads the two counter CSVs, averages each counter
             per dispatch of every kernel, scales each counter by (bytes the
             elementwise copy moves / what the counter read for it), and
             writes the per-call HBM bytes of the attention call together with
             the sha256 of the attention kernel source they were taken on. The
             factors the other calibration kernels give are recorded beside it.

    rocprofv3 --pmc FETCH_SIZE --output-format csv -d OUT_F -o p -- \\
        python3 hbm_traffic.py run
    rocprofv3 --pmc WRITE_SIZE --output-format csv -d OUT_W -o p -- \\
        python3 hbm_traffic.py run
    python3 hbm_traffic.py summarize OUT_F OUT_W \\
        profiles/attn_hbm_traffic_v3_b64_ctx8k.json
"""
import argparse
import csv
import glob
import hashlib
import json
import os
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
ATTN_SRC = os.path.join(ROOT, "kv_cache_compression_mla_amd", "csrc", "attn_mfma.hip")
COPY_BYTES = 256 << 20
KERNELS = {"attn": "attn_mfma_kernel", "combine": "combine_chunks", "copy": "MulFunctor",
           "fill": "FillFunctor", "sum": "reduce_kernel", "blit": "copyBuffer"}


def run(workload, calls):
    import torch
    from kv_cache_compression_mla_amd import inputs as gen
    from kv_cache_compression_mla_amd.step import DeviceStep
    inp = gen.make_inputs(gen.CONFIGS[workload])
    st = DeviceStep(inp)
    st.compress_append()
    st.absorb_q()
    for _ in range(calls):
        st.decode_attn()
    n = COPY_BYTES // 4
    src = torch.empty(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    acc = torch.empty(1, dtype=torch.float32, device="cuda")
    for _ in range(calls):
        src.fill_(1.0)                   # writes COPY_BYTES
        torch.mul(src, 1.0, out=dst)     # reads and writes COPY_BYTES
        torch.sum(src, 0, out=acc)       # reads COPY_BYTES
        dst.copy_(src)                   # runtime blit, COPY_BYTES each way
    torch.cuda.synchronize()
    print(f"{workload}: {calls} attention calls; {calls} x fill, copy, sum, blit of {COPY_BYTES} B", flush=True)


def _per_dispatch(directory, counter, last=5):
    """Mean counter value (summed over its instances) per dispatch, by kernel,
    over the last `last` dispatches of each (the ones `run` made)."""
    files = glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {directory}")
    per = {}
    for r in csv.DictReader(open(files[0])):
        if r["Counter_Name"] != counter:
            continue
        for key, pat in KERNELS.items():
            if pat in r["Kernel_Name"]:
                d = per.setdefault(key, {})
                d[int(r["Dispatch_Id"])] = d.get(int(r["Dispatch_Id"]), 0.0) + float(r["Counter_Value"])
    out = {}
    for k, v in per.items():
        vals = [v[i] for i in sorted(v)][-last:]
        out[k] = sum(vals) / len(vals)
    return out


def summarize(fetch_dir, write_dir, out_path, workload):
    f = _per_dispatch(fetch_dir, "FETCH_SIZE")
    w = _per_dispatch(write_dir, "WRITE_SIZE")
    # each counter in KiB; the elementwise copy moves COPY_BYTES each way
    kib = COPY_BYTES / 1024.0
    f_scale = kib / f["copy"]
    w_scale = kib / w["copy"]
    others = {"fetch_scale_from_sum": kib / f["sum"] if "sum" in f else None,
              "fetch_scale_from_blit": kib / f["blit"] if "blit" in f else None,
              "write_scale_from_fill": kib / w["fill"] if "fill" in w else None,
              "write_scale_from_blit": kib / w["blit"] if "blit" in w else None}
    parts = {}
    for k in ("attn", "combine"):
        if k in f or k in w:
            parts[k] = {"fetch_KiB_raw": f.get(k, 0.0), "write_KiB_raw": w.get(k, 0.0),
                        "fetch_bytes": f.get(k, 0.0) * f_scale * 1024.0,
                        "write_bytes": w.get(k, 0.0) * w_scale * 1024.0}
    total = sum(p["fetch_bytes"] + p["write_bytes"] for p in parts.values())
    with open(ATTN_SRC, "rb") as fh:
        sha = hashlib.sha256(fh.read()).hexdigest()
    out = {"workload": workload, "bytes_per_call": round(total),
           "kernels": parts,
           "calibration": {"kernel": "elementwise float32 copy (x * 1), 256 MiB each way",
                           "copy_bytes": COPY_BYTES, "copy_fetch_KiB_raw": f["copy"],
                           "copy_write_KiB_raw": w["copy"], "fetch_scale": f_scale, "write_scale": w_scale,
                           "other_kernels": others,
                           "raw_KiB_per_dispatch": {"FETCH_SIZE": f, "WRITE_SIZE": w}},
           "attn_source_sha256": sha,
           "commands": ["rocprofv3 --pmc FETCH_SIZE --output-format csv -d OUT_F -o p -- "
                        f"python3 hbm_traffic.py run --workload {workload}",
                        "rocprofv3 --pmc WRITE_SIZE --output-format csv -d OUT_W -o p -- "
                        f"python3 hbm_traffic.py run --workload {workload}",
                        "python3 hbm_traffic.py summarize OUT_F OUT_W OUT.json"]}
    with open(out_path, "w") as fh:
        json.dump(out, fh, indent=1)
        fh.write("\n")
    print(json.dumps(out, indent=1))


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    sub = ap.add_subparsers(dest="cmd", required=True)
    r = sub.add_parser("run")
    r.add_argument("--workload", default="v3_b64_ctx8k")
    r.add_argument("--calls", type=int, default=5)
    s = sub.add_parser("summarize")
    s.add_argument("fetch_dir")
    s.add_argument("write_dir")
    s.add_argument("out")
    s.add_argument("--workload", default="v3_b64_ctx8k")
    a = ap.parse_args()
    if a.cmd == "run":
        run(a.workload, a.calls)
    else:
        summarize(a.fetch_dir, a.write_dir, a.out, a.workload)


if __name__ == "__main__":
    sys.path.insert(0, ROOT)
    main()
