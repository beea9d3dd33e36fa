#!/usr/bin/env python3
"""Throughput of the sampling-transform scoring core on one MI355X.

One step = stce_forward + stce_backward (grad_hidden and grad_weight) over one
batch of synthetic rows at the headline shape: T = 16,384 scored tokens,
H = 5,120, V = 151,936, bf16 operands, fp32 logits, temperature 0.7,
top-k 20, top-p 0.8, targets drawn from each row's filtered distribution.

Prints one JSON line with scored tokens/s, the fraction of bf16 MFMA peak of
the whole step (8 T H V flop: forward projection, backward recompute,
hidden gradient, weight gradient), the roofline of the dominant kernel timed
with HIP events around its launches in a separate pass after the timed steps
(the timed steps themselves run with no hook attached), which filter binds
on how many rows, and the fp64 CPU oracle timed on a bounded sample of the
same rows.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0       # MI355X dense fp8 MFMA
PEAK_HBM_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def sample_targets_gpu(h, W, meta, u, chunk=1024):
    """Targets drawn from each row's filtered distribution, with plain torch
    ops on the GPU (input preparation, outside the timed region)."""
    import torch
    T = h.shape[0]
    Wf = W.float()
    out = torch.empty(T, dtype=torch.int64, device=h.device)
    uu = torch.from_numpy(u).to(h.device)
    for c0 in range(0, T, chunk):
        c1 = min(T, c0 + chunk)
        z = (h[c0:c1].float() @ Wf.T) / meta["temperature"][c0:c1, None]
        s, idx = torch.sort(z, dim=1, descending=True, stable=True)
        prob = torch.softmax(s, dim=1)
        before = torch.cumsum(prob, dim=1) - prob
        keep = before < meta["top_p"][c0:c1, None]
        keep |= (meta["top_p"][c0:c1, None] >= 1.0)
        k = meta["top_k"][c0:c1, None].long()
        ar = torch.arange(s.shape[1], device=h.device)[None, :]
        keep &= (k <= 0) | (ar < k)
        mp = meta["min_p"][c0:c1, None]
        keep &= (mp <= 0) | ((s - s[:, :1]) >= torch.log(mp.clamp_min(1e-30)))
        q = prob * keep
        cdf = torch.cumsum(q, dim=1)
        pick = torch.searchsorted(cdf, (uu[c0:c1] * cdf[:, -1]).float()[:, None].contiguous())
        pick = torch.minimum(pick, keep.sum(1, keepdim=True) - 1)
        out[c0:c1] = idx.gather(1, pick)[:, 0]
        del z, s, idx, prob, before, keep, q, cdf
    del Wf
    return out


class HipEvents:
    """Raw hipEvent_t handles for the library's per-launch timing hook."""

    def __init__(self, n):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.start = (ctypes.c_void_p * n)()
        self.stop = (ctypes.c_void_p * n)()
        for arr in (self.start, self.stop):
            for i in range(n):
                ev = ctypes.c_void_p()
                assert self.hip.hipEventCreate(ctypes.byref(ev)) == 0
                arr[i] = ev
        self.kind = (ctypes.c_int32 * n)()
        self.n = n

    def elapsed_ms(self, i):
        ms = ctypes.c_float()
        assert self.hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(self.start[i]),
                                            ctypes.c_void_p(self.stop[i])) == 0
        return ms.value


def cpu_baseline(w, y, rows):
    """fp64 oracle (as it stands) on a bounded sample of the same rows."""
    import oracle
    blas = "unknown"
    try:
        from threadpoolctl import threadpool_info
        info = threadpool_info()
        cores = max([p.get("num_threads", 1) for p in info] or [os.cpu_count()])
        blas = ", ".join(sorted({f"{p.get('internal_api')} {p.get('version')}" for p in info
                                 if p.get("user_api") == "blas"})) or blas
    except Exception:  # noqa: BLE001
        cores = os.cpu_count()
    cpu_model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), cpu_model)
    except OSError:
        pass
    sel = np.arange(rows)
    g = np.full(w["T"], -1.0 / w["T"])
    kw = dict(lane="fp8", w_scale=w["w_scale"]) if w["dtype"] == "fp8" else {}
    t0 = time.perf_counter()
    f = oracle.forward(w["h"], w["W"], y, w["temperature"], w["top_k"], w["top_p"], w["min_p"], rows=sel, **kw)
    oracle.backward(w["h"], w["W"], y, f, g, w["temperature"], w_scale=kw.get("w_scale"))
    dt = time.perf_counter() - t0
    return dict(value=rows / dt, unit="scored tokens/s", cores=int(cores), kind="oracle",
                sample=f"first {rows} rows of the same workload, forward + backward (their grad_hidden rows "
                       f"and their whole grad_weight contribution), fp64 numpy, {dt:.1f} s",
                cpu_model=cpu_model, blas=blas)


def filter_binding(info, w):
    """Rows on which each filter binds, from the forward's state: a filtered
    row whose support holds exactly top_k tokens is bound by top-k, one with
    fewer by top-p or min-p (named by which of them the workload turns on)."""
    V = w["V"]
    n = info["n"].astype(np.int64)
    k = w["top_k"].astype(np.int64)
    filt = (info["flags"] & 2) != 0
    k_on = (k > 0) & (k < V)
    out = {"unfiltered": int((~filt).sum()), "top_k": int((filt & k_on & (n == k)).sum())}
    rest = filt & ~(k_on & (n == k))
    p_on, m_on = bool((w["top_p"] < 1).any()), bool((w["min_p"] > 0).any())
    label = "top_p" if p_on and not m_on else "min_p" if m_on and not p_on else "top_p_or_min_p"
    out[label] = int(rest.sum())
    return out


def row_classes(info, g, tiled_on, nsp=128, lists=True):
    """Rows of each backward class, by the library's rule: a row with a
    gradient (target in its support, valid metadata, nonzero upstream
    gradient) is sparse when its support holds at most nsp tokens, dense
    otherwise (unfiltered rows included); a sparse row whose support the
    state lists is listed (its dz from the stored keys), else one with a
    tile list is tiled (its keys recomputed on those tiles only); the others
    are empty.  Also the (row, tile) pairs of the tiled rows."""
    fl = info["flags"]
    active = ((fl & 1) != 0) & ((fl & 4) != 0) & (g != 0)
    dense = active & (((fl & 2) == 0) | (info["n"] > nsp))
    listed = active & ~dense & ((fl & 32) != 0) & lists
    tiled = active & ~dense & ~listed & (info["ntile"] > 0) & tiled_on
    return {"dense": int(dense.sum()), "sparse": int((active & ~dense & ~listed & ~tiled).sum()),
            "listed": int(listed.sum()), "tiled": int(tiled.sum()), "empty": int((~active).sum()),
            "tile_pairs": int(info["ntile"][tiled].sum()), "entries": int(info["n"][active & ~dense].sum())}


KERNEL_SYMBOLS = {
    # kernel kind -> epilogue name in its (mangled or demangled) symbol; the bf16 main loop
    "projection": "EpiLogits",
    "dlogits": "EpiGradT<false, false>",
    "tile_recompute": "gemm_worklist",
    "grad_weight": "EpiStore",
    "grad_hidden": "EpiAccum",
    # the HBM-bound sums of the backward (their wave kernels)
    "sparse_grad_weight": "sparse_dw_wave_kernel",
    "sparse_grad_hidden": "sparse_dh_wave_kernel",
}

# kernel-trace labels: (substring of the symbol, label), first match wins
TRACE_LABELS = [
    ("EpiLogits", "gemm: forward projection + keys or candidates + tile partials (EpiLogits)"),
    ("gemm_worklist", "gemm: tile recompute of the tiled rows on their listed tiles + dz entries (EpiGrad)"),
    ("EpiGrad", "gemm: whole-vocabulary recompute + dz entries / dense dz^T (EpiGrad)"),
    ("tile_count", "tile recompute work lists (count, work items, fill)"),
    ("tile_work", "tile recompute work lists (count, work items, fill)"),
    ("tile_fill", "tile recompute work lists (count, work items, fill)"),
    ("listed_entries", "listed rows' dz entries from the state's support lists"),
    ("EpiStore", "gemm: grad_weight of the dense rows (EpiStore)"),
    ("EpiAccumT", "gemm: grad_hidden of the dense rows as dH^T (EpiAccumT)"),
    ("EpiDlogits", "gemm: backward recompute + dz^T, fp32 operands (EpiDlogits)"),
    ("sparse_dw_wave", "sparse grad_weight rows of at most 64 entries (one wave per vocabulary row)"),
    ("sparse_dw_kernel", "sparse grad_weight rows of more than 64 entries (one workgroup per vocabulary row)"),
    ("sparse_dh_wave", "sparse grad_hidden rows of at most 64 entries (one wave per row)"),
    ("sparse_dh_kernel", "sparse grad_hidden rows of more than 64 entries (one workgroup per row)"),
    ("select_kernel", "select: support program + logprob"),
    ("class_", "backward row classes (count, scan, place)"),
    ("gather_rows", "row gathers (permuted hidden rows; rows to re-project)"),
    ("bucket_fill", "dz entries filed into vocabulary-row buckets"),
    ("scan_", "exclusive scans (bucket offsets)"),
    ("transpose", "transpose (W^T, dense rows only)"),
    ("validate_kernel", "validate metadata"),
    ("fill_", "small fills (counters, status)"),
]


def mfma_busy_summary(args):
    """Writes profiles/<config>_gemm_mfma_busy.md from one `rocprofv3 --pmc
    SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CU_CYCLES GRBM_GUI_ACTIVE` run over this
    bench: per product, the clock (GRBM_GUI_ACTIVE / 8 XCDs / duration) and
    the matrix pipe's busy fraction (SQ_VALU_MFMA_BUSY_CYCLES over
    GRBM_GUI_ACTIVE / 8 x 1024 SIMDs), averaged over the launches that did
    work."""
    import csv
    import glob
    d = args.mfma_busy_summary
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    assert len(files) == 1, f"expected one counter_collection.csv in {d}, found {files}"
    disp = {}
    for r in csv.DictReader(open(files[0])):
        kn = r["Kernel_Name"]
        if "gemm_kernel" not in kn and "gemm_worklist_kernel" not in kn:
            continue
        e = disp.setdefault(r["Dispatch_Id"], {"name": kn, "id": int(r["Dispatch_Id"])})
        e[r["Counter_Name"]] = float(r["Counter_Value"])
        if "Start_Timestamp" in r and r["Start_Timestamp"]:
            e["ns"] = float(r["End_Timestamp"]) - float(r["Start_Timestamp"])
    groups = {}
    for e in disp.values():
        label = next((lab for key, lab in TRACE_LABELS if key in e["name"]), e["name"][:60])
        groups.setdefault(label, []).append(e)
    lines = [f"# Matrix-pipe busy fraction and clock per product: {args.config} fwd+bwd", "",
             "Command (from the repository root, on one MI355X):", "", "```",
             "rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CU_CYCLES GRBM_GUI_ACTIVE --output-format csv "
             f"-d <D> -- python3 bench.py --steps 1 --warmup 2 --profile-steps 1 --no-cpu-baseline --config {args.config}",
             f"python3 bench.py --mfma-busy-summary <D> --config {args.config}", "```", "",
             "clock = GRBM_GUI_ACTIVE / 8 XCDs / duration; MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / "
             "(GRBM_GUI_ACTIVE / 8 x 1024 SIMDs); averaged over the launches of the later half of the run (the "
             "counters serialize the launches). A product's launches that ran at least a quarter of its longest "
             "are its full launches; the shorter ones (re-projections of a few rows, launches with no work) are "
             "listed apart. Products none of whose launches ran a matrix instruction (above 0.05 ms) had no "
             "work (no dense rows) and are not listed.", "",
             "| product | launches | avg ms (under counters) | clock GHz | MFMA busy |", "|---|---|---|---|---|"]

    def row(label, work):
        g = np.mean([x.get("GRBM_GUI_ACTIVE", 0.0) for x in work])
        busy = np.mean([x.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / max(x.get("GRBM_GUI_ACTIVE", 1.0) / 8 * 1024, 1.0)
                        for x in work])
        ns = [x["ns"] for x in work if "ns" in x]
        ms = f"{np.mean(ns) / 1e6:.3f}" if ns else "n/a"
        clock = f"{g / 8 / np.mean(ns):.2f}" if ns else "n/a"
        lines.append(f"| {label} | {len(work)} | {ms} | {clock} | {busy:.3f} |")

    for label, es in sorted(groups.items()):
        es = sorted(es, key=lambda x: x.get("id", 0))
        es = es[len(es) // 2:] if len(es) > 1 else es                  # the later (warm) launches
        if not es or max(x.get("ns", 0.0) for x in es) < 5e4 or not any(
                x.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) > 0 for x in es):
            continue
        longest = max(x.get("ns", 0.0) for x in es)
        full = [x for x in es if x.get("ns", 0.0) >= 0.25 * longest]
        short = [x for x in es if 5e4 <= x.get("ns", 0.0) < 0.25 * longest]
        row(label, full)
        if short:
            row(label + ", short launches", short)
    lines.append("")
    out = os.path.join(ROOT, "profiles", f"{args.config}_gemm_mfma_busy.md")
    with open(out, "w") as f:
        f.write("\n".join(lines))
    print("\n".join(lines))


def kernel_stats_summary(args):
    """Writes profiles/<config>_fwd_bwd_kernel_stats.md from the
    *kernel_stats.csv of `rocprofv3 --kernel-trace --stats --output-format
    csv` over this bench."""
    import csv
    import glob
    d = args.kernel_stats_summary
    files = glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True)
    assert len(files) == 1, f"expected one kernel_stats.csv in {d}, found {files}"
    agg = {}
    total = 0.0
    for r in csv.DictReader(open(files[0])):
        ns = float(r["TotalDurationNs"])
        total += ns
        if "stce" in r["Name"]:
            label = next((lab for key, lab in TRACE_LABELS if key in r["Name"]), None)
        else:
            label = "(torch kernels of the untimed input preparation: target sampling, copies)"
        label = label or r["Name"][:80]
        a = agg.setdefault(label, [0, 0.0])
        a[0] += int(r["Calls"])
        a[1] += ns
    lines = [f"# Kernel statistics: {args.config} fwd+bwd", "",
             "Command (from the repository root, on one MI355X):", "", "```",
             f"rocprofv3 --kernel-trace --stats --output-format csv -d <D> -o {args.config} -- python3 bench.py "
             f"--steps 3 --warmup 1 --no-cpu-baseline --config {args.config}",
             f"python3 bench.py --kernel-stats-summary <D> --config {args.config}", "```", "",
             "| kernel | calls | avg ms | total ms | % of traced GPU time |", "|---|---|---|---|---|"]
    for label, (calls, ns) in sorted(agg.items(), key=lambda kv: -kv[1][1]):
        avg = f"{ns / calls / 1e6:.3f}" if calls and "torch" not in label else ""
        lines.append(f"| {label} | {calls} | {avg} | {ns / 1e6:.2f} | {100 * ns / total:.2f} |")
    n_steps = agg.get("validate metadata", (0, 0))[0]  # one metadata check per step
    lines += ["", f"The trace covers {n_steps} steps: the warm-up step, the 3 timed steps, the step with every "
              "row's keys recomputed (one untimed step and 3 timed ones; not run with --recompute-all or "
              "--fused) and the 3 steps of the per-kernel pass. Averages include the warm-up step's launches, "
              "taken while the clock ramps up.", ""]
    # the projection kernel also runs each chunk's re-projection (side stream,
    # usually no row): split its launches by stream from the kernel trace
    traces = glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True)
    if len(traces) == 1:
        rows = sorted((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), r["Stream_Id"])
                      for r in csv.DictReader(open(traces[0])) if "EpiLogits" in r["Kernel_Name"])
        if rows:
            main = rows[0][2]
            for name, sel in (("on the caller's stream (the chunks' projections)", lambda st: st == main),
                              ("on the side stream (re-projections)", lambda st: st != main)):
                ds = [(e - b) / 1e6 for b, e, st in rows if sel(st)]
                if ds:
                    lines.append(f"EpiLogits launches {name}: {len(ds)}, average {sum(ds) / len(ds):.3f} ms, "
                                 f"median {sorted(ds)[len(ds) // 2]:.3f} ms.")
            lines += ["", "A re-projection with no row to project exits at once (0.02 ms when it runs alone); one "
                      "that overlaps the next chunk's projection waits for compute-unit slots behind it, so its "
                      "span is that projection's and its work nearly none.", ""]
    out = os.path.join(ROOT, "profiles", f"{args.config}_fwd_bwd_kernel_stats.md")
    with open(out, "w") as f:
        f.write("\n".join(lines))
    print("\n".join(lines))


def source_digest():
    """sha256 over the kernel sources; a traffic figure is valid only for the
    sources it was measured on."""
    import hashlib
    d = os.path.join(ROOT, "sampling_transform_logprob_amd", "csrc")
    hsh = hashlib.sha256()
    for name in sorted(os.listdir(d)):
        if name.endswith((".hip", ".hpp", ".h")):
            hsh.update(name.encode())
            with open(os.path.join(d, name), "rb") as f:
                hsh.update(f.read())
    return hsh.hexdigest()


def traffic_file(kernel, config):
    return os.path.join(ROOT, "profiles", f"{kernel}_{config}_hbm_traffic.txt")


def read_traffic(kernel, config):
    """HBM bytes per launch of `kernel` from its committed counter summary, or
    None when there is none or the kernel sources changed since."""
    try:
        with open(traffic_file(kernel, config)) as f:
            kv = dict(line.split(":", 1) for line in f if ":" in line and not line.startswith(" "))
    except OSError:
        return None
    if kv.get("source_sha256", "").strip() != source_digest():
        return None
    return float(kv["traffic_bytes_per_launch"])


def _counter_rows(path, name_part):
    """Counter values of the dispatches of one kernel (name_part), or of the
    plain copies (name_part None), in one rocprofv3 output directory."""
    import csv
    import glob
    out = []
    files = glob.glob(os.path.join(path, "**", "*counter_collection.csv"), recursive=True)
    assert len(files) == 1, f"expected the output of one run in {path}, found {files}"
    for f in files:
        for r in csv.DictReader(open(f)):
            if name_part is None:
                if "copyBuffer" in r["Kernel_Name"]:
                    out.append(float(r["Counter_Value"]))
                continue
            kn = r["Kernel_Name"]
            gemm = ("gemm_kernel" in kn or "gemm_worklist_kernel" in kn) and "MainF32" not in kn
            if name_part in kn and (gemm or name_part.startswith("sparse_")):
                out.append(float(r["Counter_Value"]))
    # launches that did work: a re-projection with no row to project shares
    # the projection's symbol but returns at once (a counter near zero)
    if out and name_part is not None:
        big = max(out)
        out = [v for v in out if v >= 0.01 * big]
    return out


def traffic_summary(args):
    """Writes the per-launch HBM traffic of the dominant kernel from four
    rocprofv3 --pmc runs: FETCH_SIZE and WRITE_SIZE (KiB per dispatch) over
    this bench, each scaled by what the same counter reads for a plain device
    copy of known size (--copy-calibration)."""
    fetch_dir, write_dir, cfetch_dir, cwrite_dir = args.traffic_summary
    kernel, config = args.traffic_kernel, args.config
    sym = KERNEL_SYMBOLS[kernel]
    copy_sym = None
    n_copy = float(1 << 30)
    cf = _counter_rows(cfetch_dir, copy_sym)
    cw = _counter_rows(cwrite_dir, copy_sym)
    kf = _counter_rows(fetch_dir, sym)
    kw = _counter_rows(write_dir, sym)
    assert cf and cw and kf and kw, "missing dispatches in the counter output"
    # the calibration makes three copies; a copy may be split over dispatches
    cf_copy, cw_copy = sum(cf) / 3.0, sum(cw) / 3.0
    f_fac = n_copy / (cf_copy * 1024.0)     # bytes per counted KiB, reads
    w_fac = n_copy / (cw_copy * 1024.0)     # writes
    fetch_b = float(np.mean(kf)) * 1024.0 * f_fac
    write_b = float(np.mean(kw)) * 1024.0 * w_fac
    lines = [
        f"kernel: {kernel} ({sym})",
        f"workload: {config}",
        f"source_sha256: {source_digest()}",
        "commands (from the repository root, one rocprofv3 run each):",
        f"  rocprofv3 --pmc FETCH_SIZE --output-format csv -d <F> -- python3 bench.py --steps 1 --warmup 0 "
        f"--no-cpu-baseline --config {config}",
        f"  rocprofv3 --pmc WRITE_SIZE --output-format csv -d <W> -- python3 bench.py --steps 1 --warmup 0 "
        f"--no-cpu-baseline --config {config}",
        "  rocprofv3 --pmc FETCH_SIZE --output-format csv -d <CF> -- python3 bench.py --copy-calibration",
        "  rocprofv3 --pmc WRITE_SIZE --output-format csv -d <CW> -- python3 bench.py --copy-calibration",
        f"  python3 bench.py --traffic-summary <F> <W> <CF> <CW> --traffic-kernel {kernel} --config {config}",
        f"copy calibration: a 1 GiB device copy counts FETCH_SIZE {cf_copy:.0f} KiB (factor {f_fac:.4f}), "
        f"WRITE_SIZE {cw_copy:.0f} KiB (factor {w_fac:.4f})",
        f"dispatches: {len(kf)} (FETCH run), {len(kw)} (WRITE run)",
        f"FETCH_SIZE per dispatch: mean {np.mean(kf):.0f} KiB, min {min(kf):.0f}, max {max(kf):.0f}",
        f"WRITE_SIZE per dispatch: mean {np.mean(kw):.0f} KiB, min {min(kw):.0f}, max {max(kw):.0f}",
        f"fetch_bytes_per_launch: {fetch_b:.6e}",
        f"write_bytes_per_launch: {write_b:.6e}",
        f"traffic_bytes_per_launch: {fetch_b + write_b:.6e}",
        "note: FETCH_SIZE and WRITE_SIZE count L2 <-> fabric traffic, so reads served by the",
        "  Infinity Cache are included; the figure is an upper bound on HBM bytes",
    ]
    os.makedirs(os.path.dirname(traffic_file(kernel, config)), exist_ok=True)
    with open(traffic_file(kernel, config), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def copy_calibration():
    """A plain device-to-device copy of 1 GiB, three times (counter scale)."""
    import torch
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "launches": 3}), flush=True)


def library_reference(reps=5):
    """The four products of the step at the headline shape, each as one
    torch.mm call (the vendor library, hipBLASLt on ROCm) on synthetic bf16
    operands of the same layouts, with bf16 and with fp32 output: a reference
    rate for the matrix products alone, without the path's epilogues
    (temperature, tile partials, keys, dz).  Not part of the scoring path."""
    import torch
    T, H, V, C = 16384, 5120, 151936, 4096
    g = torch.Generator(device="cuda").manual_seed(0)
    W = (torch.randn(V, H, device="cuda", generator=g) * 0.02).to(torch.bfloat16)
    h = torch.randn(T, H, device="cuda", generator=g).to(torch.bfloat16)
    dT = (torch.randn(V, T, device="cuda", generator=g) * 1e-6).to(torch.bfloat16)
    products = [
        ("projection z^T = W h_chunk^T (K = H)", lambda dt: torch.mm(W, h[:C].t(), out_dtype=dt), V * C * H),
        ("recompute z^T = W h^T (K = H)", lambda dt: torch.mm(W, h.t(), out_dtype=dt), V * T * H),
        ("grad_weight dW = dz^T h (K = T)", lambda dt: torch.mm(dT, h, out_dtype=dt), V * H * T),
        ("grad_hidden dH^T = W^T dz^T (K = V)", lambda dt: torch.mm(W.t(), dT, out_dtype=dt), H * T * V),
    ]
    out = []
    for name, f, mnk in products:
        for dt in (torch.bfloat16, torch.float32):
            f(dt)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                r = f(dt)
            e1.record()
            torch.cuda.synchronize()
            del r
            ms = e0.elapsed_time(e1) / reps
            tf = 2.0 * mnk / (ms * 1e-3) / 1e12
            out.append(dict(product=name, out_dtype=str(dt).replace("torch.", ""), ms=ms, tflops=tf))
            log(f"[library] {name:40s} out {out[-1]['out_dtype']:8s} {ms:8.3f} ms {tf:7.1f} TFLOP/s")
    print(json.dumps({"library_reference": out}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="headline")
    ap.add_argument("--cpu-rows", type=int, default=None,
                    help="rows of the CPU oracle's sample (default 512; 256 in the fp8 lane, whose oracle also "
                         "decodes the whole e4m3 weight in fp64): about 10-30 s of CPU work")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile-steps", type=int, default=3,
                    help="steps of the separate pass that records HIP events around each launch")
    ap.add_argument("--chunk-rows", type=int, default=0)
    ap.add_argument("--vocab-slice", type=int, default=0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run a plain 1 GiB device copy (scale of the HBM byte counters) and exit")
    ap.add_argument("--traffic-summary", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR"),
                    help="write the HBM traffic summary of --traffic-kernel from rocprofv3 --pmc outputs and exit")
    ap.add_argument("--traffic-kernel", default="projection")
    ap.add_argument("--mfma-busy-summary", metavar="DIR",
                    help="write the matrix-pipe busy summary of --config from a rocprofv3 --pmc csv output "
                         "directory and exit")
    ap.add_argument("--kernel-stats-summary", metavar="DIR",
                    help="write the kernel statistics summary of --config from a rocprofv3 --stats csv output "
                         "directory and exit")
    ap.add_argument("--library-reference", action="store_true",
                    help="time the step's four products as plain torch.mm calls (vendor library) and exit")
    ap.add_argument("--side-outputs", action="store_true",
                    help="forward with the sweep's side outputs (full LSE, full and support entropy)")
    ap.add_argument("--policy-loss", choices=["none", "cispo", "clip"], default="none",
                    help="time the fused policy-gradient step instead: forward, per-token loss (advantages "
                         "and behaviour logprobs synthetic), backward of the summed loss")
    ap.add_argument("--fused", action="store_true",
                    help="with --policy-loss: the fused step (dlogits formed in the forward's sweep from the "
                         "chunk's keys, 3 products instead of 4)")
    ap.add_argument("--lane", choices=["fp32", "bf16"], default="fp32",
                    help="bf16: the bf16 value lane (bf16 keys, bf16 logprob)")
    ap.add_argument("--pre-gemm-temperature", type=float, default=None,
                    help="one scalar temperature applied to the hidden states before the projection, in place "
                         "of the workload's per-row temperature applied after it")
    ap.add_argument("--recompute-all", action="store_true",
                    help="the backward recomputes every row's keys (the recompute closed-form VJP for every row), "
                         "ignoring the support lists the forward keeps in the state")
    args = ap.parse_args()
    if args.fused and args.policy_loss == "none":
        print("--fused needs --policy-loss cispo|clip", file=sys.stderr)
        sys.exit(2)
    if args.traffic_summary:
        traffic_summary(args)
        return
    if args.kernel_stats_summary:
        kernel_stats_summary(args)
        return
    if args.mfma_busy_summary:
        mfma_busy_summary(args)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (this build has no multi-GPU path); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration:
        copy_calibration()
        return
    if args.library_reference:
        library_reference()
        return

    import torch

    from sampling_transform_logprob_amd import binding, workloads
    L = binding.load()
    dev = torch.device("cuda:0")

    log(f"[bench] generating {args.config} inputs")
    w = workloads.make(args.config)
    T, H, V = w["T"], w["H"], w["V"]
    fp8 = w["dtype"] == "fp8"
    dt = torch.float32 if w["dtype"] == "f32" else torch.bfloat16
    h = torch.from_numpy(w["h"]).to(dev).to(dt)
    W = torch.from_numpy(w["W"]).to(dev) if fp8 else torch.from_numpy(w["W"]).to(dev).to(dt)
    w_scale = torch.from_numpy(w["w_scale"]).to(dev) if fp8 else None
    meta = dict(temperature=torch.from_numpy(w["temperature"]).to(dev), top_k=torch.from_numpy(w["top_k"]).to(dev),
                top_p=torch.from_numpy(w["top_p"]).to(dev), min_p=torch.from_numpy(w["min_p"]).to(dev))
    log("[bench] drawing targets from the filtered distributions")
    if w["filtered"] and fp8:
        # input preparation with torch's own e4m3 conversion: the dequantized
        # operands of the lane (rows of h scaled by amax / 448)
        a = (h.float().abs().amax(1, keepdim=True) / 448.0).clamp_min(1e-30)
        h_deq = (h.float() / a).clamp(-448, 448).to(torch.float8_e4m3fn).float() * a
        W_deq = W.view(torch.float8_e4m3fn).float() * w_scale[:, None]
        target = sample_targets_gpu(h_deq, W_deq, meta, w["u"])
        del h_deq, W_deq
    elif w["filtered"]:
        target = sample_targets_gpu(h, W, meta, w["u"])
    else:
        target = torch.from_numpy(w["target_uniform"]).to(dev)
    torch.cuda.synchronize()

    ts = args.pre_gemm_temperature
    prob, keep = binding.make_problem(h, W, target, None if ts is not None else meta["temperature"], meta["top_k"],
                                      meta["top_p"], meta["min_p"], args.chunk_rows, args.vocab_slice,
                                      pre_gemm_temperature=ts, lane=args.lane, weight_scale=w_scale,
                                      recompute_all=args.recompute_all)
    fwd_b, bwd_b = binding.workspace_bytes(prob)
    ws_f = torch.empty(fwd_b, dtype=torch.uint8, device=dev)
    ws_b = torch.empty(bwd_b, dtype=torch.uint8, device=dev)
    logprob = torch.empty(T, dtype=torch.float32, device=dev)
    state = torch.empty(T * binding.STATE_BYTES_PER_ROW, dtype=torch.uint8, device=dev)
    gh = torch.empty(T, H, dtype=dt, device=dev)
    gw = torch.empty(V, H, dtype=torch.float32, device=dev)
    g = torch.full((T,), -1.0 / T, dtype=torch.float32, device=dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    P = ctypes.byref(prob)
    pg = None
    if args.policy_loss != "none":
        # synthetic advantages and behaviour logprobs (seeded), fp32 on the device
        rng = np.random.Generator(np.random.PCG64(17))
        adv = torch.from_numpy(rng.standard_normal(T).astype(np.float32)).to(dev)
        old_lp = torch.from_numpy((-rng.exponential(1.0, T)).astype(np.float32)).to(dev)
        loss_t = torch.empty(T, dtype=torch.float32, device=dev)
        pg = binding.PgParams(binding.PG_OBJECTIVES[args.policy_loss], 0.2, 0.28, 1.0 / T, adv.data_ptr(),
                              old_lp.data_ptr())

    side = None
    if args.side_outputs:
        side_t = [torch.empty(T, dtype=torch.float32, device=dev) for _ in range(3)]
        side = binding.SideOutputs(*(t.data_ptr() for t in side_t))
    if args.fused:
        del ws_f, ws_b
        fus_b, _ = binding.fused_workspace_bytes(prob)
        ws_u = torch.empty(fus_b, dtype=torch.uint8, device=dev)

    def fused_step():
        binding._check(L.stce_fused_policy_step(
            P, ctypes.byref(pg), ctypes.c_void_p(logprob.data_ptr()), ctypes.c_void_p(state.data_ptr()),
            ctypes.c_void_p(loss_t.data_ptr()), None, None if side is None else ctypes.byref(side),
            ctypes.c_void_p(gh.data_ptr()), ctypes.c_void_p(gw.data_ptr()), 0, None,
            ctypes.c_void_p(ws_u.data_ptr()), fus_b, stream))

    def step():
        if args.fused:
            fused_step()
            return
        if side is not None:
            binding._check(L.stce_forward_with_side(P, ctypes.c_void_p(logprob.data_ptr()),
                                                    ctypes.c_void_p(state.data_ptr()), ctypes.byref(side), None,
                                                    ctypes.c_void_p(ws_f.data_ptr()), fwd_b, stream))
        else:
            binding._check(L.stce_forward(P, ctypes.c_void_p(logprob.data_ptr()), ctypes.c_void_p(state.data_ptr()),
                                          None, ctypes.c_void_p(ws_f.data_ptr()), fwd_b, stream))
        if pg is not None:
            binding._check(L.stce_policy_loss(ctypes.byref(pg), T, ctypes.c_void_p(logprob.data_ptr()),
                                              ctypes.c_void_p(loss_t.data_ptr()), ctypes.c_void_p(g.data_ptr()),
                                              None, stream))
        binding._check(L.stce_backward(P, ctypes.c_void_p(g.data_ptr()), ctypes.c_void_p(state.data_ptr()),
                                       ctypes.c_void_p(gh.data_ptr()), ctypes.c_void_p(gw.data_ptr()), 0, None,
                                       ctypes.c_void_p(ws_b.data_ptr()), bwd_b, stream))

    log(f"[bench] warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    in_support = float((logprob > -float("inf")).float().mean().item())
    binds = filter_binding(binding.decode_state(state), w)
    log(f"[bench] binding filter per row: {binds}")

    # the headline figure: K steps with no profiling hook attached
    log(f"[bench] timing {args.steps} steps")
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    t_start.record()
    for i in range(args.steps):
        marks[i].record()
        step()
    marks[args.steps].record()
    t_end.record()
    torch.cuda.synchronize()
    ms_step = t_start.elapsed_time(t_end) / args.steps
    per_step = np.array([marks[i].elapsed_time(marks[i + 1]) for i in range(args.steps)])

    # the same step with every row's keys recomputed (the support lists the
    # state holds unused): the recompute closed-form VJP for every row, timed
    # apart so that the line carries both
    recompute_all = None
    if not args.fused and not args.recompute_all and dt == torch.bfloat16:
        prob_r, keep_r = binding.make_problem(h, W, target, None if ts is not None else meta["temperature"],
                                              meta["top_k"], meta["top_p"], meta["min_p"], args.chunk_rows,
                                              args.vocab_slice, pre_gemm_temperature=ts, lane=args.lane,
                                              weight_scale=w_scale, recompute_all=True)
        P_main, P = P, ctypes.byref(prob_r)
        n_r = max(1, min(args.steps, 10))
        step()
        r_start, r_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        r_start.record()
        for _ in range(n_r):
            step()
        r_end.record()
        torch.cuda.synchronize()
        P = P_main
        ms_r = r_start.elapsed_time(r_end) / n_r
        recompute_all = {"ms_per_step": ms_r, "value": T / (ms_r * 1e-3), "steps": n_r}
        log(f"[bench] with every row recomputed: {ms_r:.3f} ms per step over {n_r} steps")

    # per-kernel figures: a separate pass with HIP events recorded around each
    # launch on its stream (stce_profile_attach)
    prof_steps = max(1, min(args.steps, args.profile_steps))
    ev = HipEvents(256 * prof_steps)
    prof = binding.Profile(ev.n, 0, ctypes.cast(ev.start, ctypes.POINTER(ctypes.c_void_p)),
                           ctypes.cast(ev.stop, ctypes.POINTER(ctypes.c_void_p)),
                           ctypes.cast(ev.kind, ctypes.POINTER(ctypes.c_int32)))
    log(f"[bench] per-kernel pass: {prof_steps} steps with launch events")
    p_start = torch.cuda.Event(enable_timing=True)
    p_end = torch.cuda.Event(enable_timing=True)
    L.stce_profile_attach(ctypes.byref(prof))
    torch.cuda.synchronize()
    p_start.record()
    for i in range(prof_steps):
        step()
    p_end.record()
    torch.cuda.synchronize()
    L.stce_profile_attach(None)
    ms_step_profiled = p_start.elapsed_time(p_end) / prof_steps

    # per-kind launch statistics from the events recorded around each launch
    kinds = {}
    for i in range(prof.count):
        k = binding.KERNEL_KINDS.get(ev.kind[i], str(ev.kind[i]))
        kinds.setdefault(k, []).append(ev.elapsed_ms(i))
    # algorithmic flop per launch of each product: each kind of product does
    # 2 T H V per step (the fused step has no dlogits product), spread over
    # the launches observed
    C, Vs = binding.schedule(prob)
    # the fused step's path: with row classes for bf16 operands with a filter
    # and for the fp8 lane, dense otherwise
    any_filter = any(meta[k] is not None for k in ("top_k", "top_p", "min_p"))
    fused_classed = args.fused and dt == torch.bfloat16 and (fp8 or any_filter)
    if args.fused and not fused_classed:
        C = min(-(-(args.chunk_rows or 4096) // 64) * 64, -(-T // 64) * 64)
        Vs = None
    # the backward's row classes (bf16 and the fp8 lane): the recompute
    # product runs over the rows with a gradient, the two gradient products
    # over the dense rows; sparse rows' gradients are sums over their dz
    # entries, formed from the keys the state lists, or recomputed on their
    # listed tiles, or in the whole-vocabulary recompute
    classed = dt == torch.bfloat16 and (not args.fused or fused_classed)
    tiled_on = classed and -(-V // 256) <= 65535 and T * H * (1 if fp8 else 2) < 2 ** 31 - 1 - 2 ** 22
    classes = row_classes(binding.decode_state(state), g.cpu().numpy(), tiled_on, lists=not args.recompute_all)
    t_full = classes["dense"] + classes["sparse"] if classed else T
    t_dense = classes["dense"] if classed else T
    # the tile recompute forms 256 keys of H-long products per (row, tile) pair
    per_step_flop = {"projection": 2.0 * T * H * V, "dlogits": 2.0 * t_full * H * V,
                     "tile_recompute": 2.0 * classes["tile_pairs"] * 256 * H if classed else 0.0,
                     "grad_weight": 2.0 * t_dense * H * V, "grad_hidden": 2.0 * t_dense * H * V}
    if args.fused and not fused_classed:
        per_step_flop = {k: 2.0 * T * H * V for k in ("projection", "grad_weight", "grad_hidden")}
    stats = {}
    per_launch = {}
    for k, v in kinds.items():
        a = np.array(v)
        n_launch = len(a) / prof_steps
        stats[k] = dict(launches=int(n_launch), avg_ms=float(a.mean()), total_ms_per_step=float(a.sum() / prof_steps))
        if per_step_flop.get(k):
            per_launch[k] = per_step_flop[k] / n_launch
            stats[k]["tflops"] = per_launch[k] / (a.mean() * 1e-3) / 1e12
    if "reproject" in stats:
        # its events are recorded on the side stream, where each launch waits
        # for compute-unit slots behind the next chunk's projection: the span
        # is mostly that projection's, the work only the chunk's undecided rows
        stats["reproject"]["note"] = ("side-stream span, overlapping the next projection; work only for rows "
                                      "the candidates could not decide")
    if "select" in stats:
        stats["select"]["note"] = "side stream, overlapping the next chunk's projection except after the last chunk"
    dom = max((k for k in stats if k in per_launch), key=lambda k: stats[k]["total_ms_per_step"])
    achieved = stats[dom]["tflops"]
    # the fp8 lane's projection and recompute run on e4m3 operands (the fp8
    # peak), its two gradient products on bf16 ones
    peak_of = {k: (PEAK_FP8_TFLOPS if fp8 and k in ("projection", "dlogits", "tile_recompute") else PEAK_BF16_TFLOPS)
               for k in per_step_flop}
    t_at_peak = sum(f / (peak_of[k] * 1e12) for k, f in per_step_flop.items())

    # the backward's HBM-bound sums: algorithmic bytes of a launch over its
    # average duration, against the 8 TB/s peak (E dz entries of the sparse
    # rows: dW writes every fp32 row and gathers a hidden row per entry, dH
    # gathers a weight row per entry and writes the non-dense rows)
    hbm_kernels = {}
    if classed:
        E, T_sp = classes["entries"], T - classes["dense"]
        ew = 1 if fp8 else 2
        algo = {"sparse_grad_weight": 4.0 * V * H + 2.0 * E * H + 24.0 * E,
                "sparse_grad_hidden": float(ew) * E * H + 2.0 * T_sp * H + 8.0 * E,
                "listed_entries": 16.0 * E}
        for k, b in algo.items():
            if k in stats:
                per = b / stats[k]["launches"]
                gbs = per / (stats[k]["avg_ms"] * 1e-3) / 1e9
                hbm_kernels[k] = {"bound": "hbm", "bytes_per_launch": per, "achieved": gbs, "peak": PEAK_HBM_GBS,
                                  "unit": "GB/s", "frac": gbs / PEAK_HBM_GBS, "traffic": read_traffic(k, args.config)}

    # matrix-core flop the step performs (the dense formulation would perform
    # 8 T H V: forward, recompute, dH, dW over every row)
    flop_step = sum(per_step_flop.values())
    value = T / (ms_step * 1e-3)
    out = {
        "metric": "scored tokens/s fwd+bwd at V=151936,H=5120; % of bf16 MFMA peak",
        "value": value,
        "unit": "scored tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "ms_per_step_median": float(np.median(per_step)),
        "ms_per_step_min": float(per_step.min()),
        "ms_per_step_with_launch_events": ms_step_profiled,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8" if fp8 else "bf16" if dt == torch.bfloat16 else "f32",
        "data": ("synthetic (seeded PCG64; h ~ N(0,1) bf16; W e4m3 codes drawn as bit fields, exponent field "
                 "14 - Geometric(1/2), uniform mantissa and sign, row scales 1.4e-4 * 2^U(-1/2, 1/2); targets drawn "
                 "from the filtered distributions)" if fp8 else
                 "synthetic (seeded PCG64; h ~ N(0,1), W ~ N(0,0.02^2), bf16; targets drawn from the filtered "
                 "distributions)"),
        "config": {"workload": f"{args.config}: T={T} scored tokens, H={H}, V={V}, temperature "
                               f"{'per-row' if args.config != 'headline' else 0.7}, top_k "
                               f"{int(w['top_k'].max())}, top_p {float(w['top_p'].min())}, min_p "
                               f"{float(w['min_p'].max())}; forward + backward (grad_hidden, grad_weight)"
                               + ("" if args.policy_loss == "none" else
                                  f" of the {args.policy_loss} policy-gradient token loss")
                               + ("; fused step (forward, loss and backward in one call)" if fused_classed else
                                  "; fused step: dlogits formed in the forward's sweep, no recompute product"
                                  if args.fused else "")
                               + ("; forward side outputs (full LSE, entropies)" if args.side_outputs else "")
                               + ("; bf16 value lane" if args.lane == "bf16" else "")
                               + ("; fp8 lane: e4m3 weight with per-row scales, hidden rows quantized per row, "
                                  "logits and recompute on fp8 matrix cores, gradient products bf16" if fp8 else "")
                               + (f"; scalar pre-GEMM temperature {ts} in place of the per-row one"
                                  if ts is not None else "")
                               + ("; every row's keys recomputed (support lists unused)" if args.recompute_all
                                  else ""),
                   "T": T, "H": H, "V": V, "chunk_rows": C, "vocab_slice": Vs},
        "mfma_peak_frac": t_at_peak / (ms_step * 1e-3),
        "mfma_flop_per_step": flop_step,
        "tflops_performed": flop_step / (ms_step * 1e-3) / 1e12,
        "tflops_8thv": 8.0 * T * H * V / (ms_step * 1e-3) / 1e12,
        "dense_equivalent_frac_8thv": 8.0 * T * H * V / (ms_step * 1e-3) / (PEAK_BF16_TFLOPS * 1e12),
        "tflops_6thv": 6.0 * T * H * V / (ms_step * 1e-3) / 1e12,
        "row_classes": classes if classed else None,
        "roofline": {"kernel": dom, "bound": "mfma", "achieved": achieved, "peak": peak_of[dom],
                     "unit": "TFLOP/s", "frac": achieved / peak_of[dom],
                     "traffic": read_traffic(dom, args.config)},
        "kernels": stats,
        "hbm_kernels": hbm_kernels,
        "recompute_all": recompute_all,
        "targets_in_support": in_support,
        "binding_filter_rows": binds,
    }
    if not args.no_cpu_baseline:
        rows = args.cpu_rows or (256 if fp8 else 512)
        log(f"[bench] cpu baseline: oracle on {rows} rows")
        w_np = dict(w)
        out["cpu_baseline"] = cpu_baseline(w_np, target.cpu().numpy(), rows)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
