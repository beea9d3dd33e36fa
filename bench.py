#!/usr/bin/env python3
"""Throughput of the sampling-transform scoring core on one MI355X.

One step = stce_forward + stce_backward (grad_hidden and grad_weight) over one
batch of synthetic rows at the headline shape: T = 16,384 scored tokens,
H = 5,120, V = 151,936, bf16 operands, fp32 logits, temperature 0.7,
top-k 20, top-p 0.8, targets drawn from each row's filtered distribution.

Prints one JSON line with scored tokens/s, the fraction of bf16 MFMA peak of
the whole step (8 T H V flop: forward projection, backward recompute,
hidden gradient, weight gradient), the roofline of the dominant kernel timed
with HIP events around its launches inside the timed steps, and the fp64 CPU
oracle timed on a bounded sample of the same rows.
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
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [os.cpu_count()])
    except Exception:  # noqa: BLE001
        cores = os.cpu_count()
    sel = np.arange(rows)
    g = np.full(w["T"], -1.0 / w["T"])
    t0 = time.perf_counter()
    f = oracle.forward(w["h"], w["W"], y, w["temperature"], w["top_k"], w["top_p"], w["min_p"], rows=sel)
    oracle.backward(w["h"], w["W"], y, f, g, w["temperature"])
    dt = time.perf_counter() - t0
    return dict(value=rows / dt, unit="scored tokens/s", cores=int(cores), kind="oracle",
                sample=f"first {rows} rows of the same workload, forward + backward (their grad_hidden rows "
                       f"and their whole grad_weight contribution), fp64 numpy, {dt:.1f} s")


KERNEL_SYMBOLS = {
    # kernel kind -> epilogue name in its (mangled or demangled) symbol; the bf16 main loop
    "projection": "EpiLogits",
    "dlogits": "EpiDlogits",
    "grad_weight": "EpiStore",
    "grad_hidden": "EpiAccum",
}


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
            if name_part in kn and "gemm_kernel" in kn and "MainBf16" in kn:
                out.append(float(r["Counter_Value"]))
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
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="headline")
    ap.add_argument("--cpu-rows", type=int, default=512)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--chunk-rows", type=int, default=0)
    ap.add_argument("--vocab-slice", type=int, default=0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run a plain 1 GiB device copy (scale of the HBM byte counters) and exit")
    ap.add_argument("--traffic-summary", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR"),
                    help="write the HBM traffic summary of --traffic-kernel from rocprofv3 --pmc outputs and exit")
    ap.add_argument("--traffic-kernel", default="dlogits")
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
    args = ap.parse_args()
    if args.fused and args.policy_loss == "none":
        print("--fused needs --policy-loss cispo|clip", file=sys.stderr)
        sys.exit(2)
    if args.traffic_summary:
        traffic_summary(args)
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
    dt = torch.float32 if w["dtype"] == "f32" else torch.bfloat16
    h = torch.from_numpy(w["h"]).to(dev).to(dt)
    W = torch.from_numpy(w["W"]).to(dev).to(dt)
    meta = dict(temperature=torch.from_numpy(w["temperature"]).to(dev), top_k=torch.from_numpy(w["top_k"]).to(dev),
                top_p=torch.from_numpy(w["top_p"]).to(dev), min_p=torch.from_numpy(w["min_p"]).to(dev))
    log("[bench] drawing targets from the filtered distributions")
    if w["filtered"]:
        target = sample_targets_gpu(h, W, meta, w["u"])
    else:
        target = torch.from_numpy(w["target_uniform"]).to(dev)
    torch.cuda.synchronize()

    ts = args.pre_gemm_temperature
    prob, keep = binding.make_problem(h, W, target, None if ts is not None else meta["temperature"], meta["top_k"],
                                      meta["top_p"], meta["min_p"], args.chunk_rows, args.vocab_slice,
                                      pre_gemm_temperature=ts, lane=args.lane)
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

    ev = HipEvents(256 * max(args.steps, 1))
    prof = binding.Profile(ev.n, 0, ctypes.cast(ev.start, ctypes.POINTER(ctypes.c_void_p)),
                           ctypes.cast(ev.stop, ctypes.POINTER(ctypes.c_void_p)),
                           ctypes.cast(ev.kind, ctypes.POINTER(ctypes.c_int32)))
    log(f"[bench] timing {args.steps} steps")
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    L.stce_profile_attach(ctypes.byref(prof))
    torch.cuda.synchronize()
    t_start.record()
    for i in range(args.steps):
        marks[i].record()
        step()
    marks[args.steps].record()
    t_end.record()
    torch.cuda.synchronize()
    L.stce_profile_attach(None)
    ms_step = t_start.elapsed_time(t_end) / args.steps
    per_step = np.array([marks[i].elapsed_time(marks[i + 1]) for i in range(args.steps)])

    # per-kind launch statistics from the events recorded around each launch
    kinds = {}
    for i in range(prof.count):
        k = binding.KERNEL_KINDS.get(ev.kind[i], str(ev.kind[i]))
        kinds.setdefault(k, []).append(ev.elapsed_ms(i))
    # algorithmic flop per launch of each product: each kind of product does
    # 2 T H V per step (the fused step has no dlogits product), spread over
    # the launches observed
    C, Vs = binding.schedule(prob)
    if args.fused:
        C = min(-(-(args.chunk_rows or 4096) // 64) * 64, -(-T // 64) * 64)
        Vs = None
    per_step_flop = {k: 2.0 * T * H * V for k in ("projection", "dlogits", "grad_weight", "grad_hidden")}
    stats = {}
    per_launch = {}
    for k, v in kinds.items():
        a = np.array(v)
        n_launch = len(a) / args.steps
        stats[k] = dict(launches=int(n_launch), avg_ms=float(a.mean()), total_ms_per_step=float(a.sum() / args.steps))
        if k in per_step_flop:
            per_launch[k] = per_step_flop[k] / n_launch
            stats[k]["tflops"] = per_launch[k] / (a.mean() * 1e-3) / 1e12
    dom = max((k for k in stats if k in per_launch), key=lambda k: stats[k]["total_ms_per_step"])
    achieved = stats[dom]["tflops"]

    flop_step = (6.0 if args.fused else 8.0) * T * H * V
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
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if dt == torch.bfloat16 else "f32",
        "data": "synthetic (seeded PCG64; h ~ N(0,1), W ~ N(0,0.02^2), bf16; targets drawn from the filtered "
                "distributions)",
        "config": {"workload": f"{args.config}: T={T} scored tokens, H={H}, V={V}, temperature "
                               f"{'per-row' if args.config != 'headline' else 0.7}, top_k "
                               f"{int(w['top_k'].max())}, top_p {float(w['top_p'].min())}, min_p "
                               f"{float(w['min_p'].max())}; forward + backward (grad_hidden, grad_weight)"
                               + ("" if args.policy_loss == "none" else
                                  f" of the {args.policy_loss} policy-gradient token loss")
                               + ("; fused step: dlogits formed in the forward's sweep, no recompute product"
                                  if args.fused else "")
                               + ("; forward side outputs (full LSE, entropies)" if args.side_outputs else "")
                               + ("; bf16 value lane" if args.lane == "bf16" else "")
                               + (f"; scalar pre-GEMM temperature {ts} in place of the per-row one"
                                  if ts is not None else ""),
                   "T": T, "H": H, "V": V, "chunk_rows": C, "vocab_slice": Vs},
        "mfma_peak_frac": flop_step / (ms_step * 1e-3) / (PEAK_BF16_TFLOPS * 1e12),
        "tflops_8thv": 8.0 * T * H * V / (ms_step * 1e-3) / 1e12,
        "tflops_performed": flop_step / (ms_step * 1e-3) / 1e12,
        "tflops_6thv": 6.0 * T * H * V / (ms_step * 1e-3) / 1e12,
        "roofline": {"kernel": dom, "bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                     "traffic": read_traffic(dom, args.config)},
        "kernels": stats,
        "targets_in_support": in_support,
    }
    if not args.no_cpu_baseline:
        log(f"[bench] cpu baseline: oracle on {args.cpu_rows} rows")
        w_np = dict(w)
        out["cpu_baseline"] = cpu_baseline(w_np, target.cpu().numpy(), args.cpu_rows)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
