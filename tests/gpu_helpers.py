"""Shared helpers of the GPU parity tests: build seeded inputs, run the HIP
path through the C ABI, run the oracle on the same inputs and compare.

The bar (the support must match bit for bit on identical fp32 keys; logprob
within 2e-3 absolute; gradients within 1e-2 relative Frobenius error) is the
one the scoring core is held to."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
from sampling_transform_logprob_amd import binding, workloads

LOGPROB_ATOL = 2e-3
GRAD_RTOL = 1e-2


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev():
    return torch.device("cuda:0")


def to_gpu(w, y):
    dt = torch.float32 if w["dtype"] == "f32" else torch.bfloat16
    d = dev()
    fp8 = w["dtype"] == "fp8"
    out = dict(
        h=torch.from_numpy(w["h"]).to(d).to(dt),
        W=torch.from_numpy(w["W"]).to(d) if fp8 else torch.from_numpy(w["W"]).to(d).to(dt),
        target=torch.from_numpy(np.asarray(y, np.int64)).to(d),
        temperature=torch.from_numpy(w["temperature"]).to(d), top_k=torch.from_numpy(w["top_k"]).to(d),
        top_p=torch.from_numpy(w["top_p"]).to(d), min_p=torch.from_numpy(w["min_p"]).to(d))
    out["weight_scale"] = torch.from_numpy(w["w_scale"]).to(d) if fp8 else None
    return out


def lane_of(w):
    """The oracle's lane name and keyword arguments for a workload."""
    return ("fp8", dict(w_scale=w["w_scale"])) if w["dtype"] == "fp8" else ("fp32", {})


def targets(w, rows=None):
    if not w["filtered"]:
        return w["target_uniform"] if rows is None else w["target_uniform"][rows]
    lane, kw = lane_of(w)
    return oracle.sample_targets(w["h"], w["W"], w["temperature"], w["top_k"], w["top_p"], w["min_p"], w["u"],
                                 rows=rows, lane=lane, **kw)


def meta_of(g):
    return {k: g[k] for k in ("temperature", "top_k", "top_p", "min_p")}


def rel_fro(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    nb = np.linalg.norm(b)
    return np.linalg.norm(a - b) / (nb if nb > 0 else 1.0)


def check_support(info, ref, rows_label=""):
    """Bit-exact support on identical keys (rows the oracle flags as within
    rounding of a decision are reported and excluded)."""
    near = ref["near"]
    ok = ~near
    assert np.array_equal(info["n"][ok], ref["n"][ok]), (
        f"{rows_label} support size mismatch at rows {np.nonzero((info['n'] != ref['n']) & ok)[0][:10]}")
    # unfiltered rows keep the sentinel boundary (0, V - 1); filtered rows
    # keep the last support token, which must be the oracle's
    filt = ((info["flags"] & binding.FLAG_FILTERED) != 0) & ok
    bad = filt & ((info["key_thr"] != ref["key_thr"]) | (info["id_thr"] != ref["id_thr"]))
    assert not bad.any(), f"{rows_label} boundary mismatch at rows {np.nonzero(bad)[0][:10]}"
    return int(near.sum())


def check_logprob(lp_gpu, ref):
    lp = np.asarray(lp_gpu, np.float64)
    fin = np.isfinite(ref["logprob"])
    assert np.array_equal(np.isfinite(lp), fin), "in/out-of-support pattern differs"
    assert np.all(lp[~fin] == -np.inf)
    err = float(np.abs(lp[fin] - ref["logprob"][fin]).max()) if fin.any() else 0.0
    assert err < LOGPROB_ATOL, f"logprob max abs error {err}"
    return err
