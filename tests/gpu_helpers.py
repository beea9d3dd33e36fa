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


NSP = 128


def _sparse_rows(info, g):
    fl = info["flags"]
    ok = ((fl & binding.FLAG_VALID) != 0) & ((fl & binding.FLAG_IN_SUPPORT) != 0) & (np.asarray(g) != 0)
    return ok & ((fl & binding.FLAG_FILTERED) != 0) & (info["n"] <= NSP)


def listed_rows(info, g, dtype):
    """Rows whose dz the backward forms from the support the state lists (the
    library's class rule): valid, target in support, filtered, at most NSP
    support tokens, nonzero upstream gradient, the listed flag, bf16 or fp8
    operands."""
    return _sparse_rows(info, g) & ((info["flags"] & binding.FLAG_LISTED) != 0) & (dtype != "f32")


def tiled_rows(info, g, V, dtype):
    """Rows whose keys the backward recomputes on their listed tiles only (the
    library's class rule): as listed_rows but with no support list, and a
    tile list."""
    return (_sparse_rows(info, g) & ((info["flags"] & binding.FLAG_LISTED) == 0) & (info["ntile"] > 0)
            & (dtype != "f32") & (-(-V // 256) <= 65535))


def unlisted(st, T):
    """A copy of a state with every row's listed flag cleared: the backward
    then takes those rows' keys from the recompute again."""
    s = st.clone()
    rec = s[: T * binding.RECORD_BYTES].view(torch.int32).view(T, 8)
    rec[:, 3] &= ~binding.FLAG_LISTED
    return s


def without_lists(st, T):
    """A copy of a state with neither tile lists nor support lists: every
    sparse row goes through the whole-vocabulary recompute."""
    s = unlisted(st, T)
    s[T * binding.RECORD_BYTES:] = 0
    return s


def check_support_lists(info, keys):
    """A listed row's support list holds its n support tokens in decreasing
    (key, -id) order with the forward's keys bit for bit, and zeros after;
    every other row's list is zero."""
    T = keys.shape[0]
    listed = (info["flags"] & binding.FLAG_LISTED) != 0
    for r in range(T):
        ids, ks = info["support_ids"][r], info["support_keys"][r]
        if not listed[r]:
            assert not ids.any() and not ks.view(np.int32).any(), r
            continue
        n = int(info["n"][r])
        assert n <= NSP and (info["flags"][r] & binding.FLAG_FILTERED), r
        row = keys[r]
        kthr, ithr = row[info["id_thr"][r]], info["id_thr"][r]
        idx = np.arange(row.shape[0])
        want = np.nonzero((row > kthr) | ((row == kthr) & (idx <= ithr)))[0]
        want = want[np.lexsort((want, -row[want].astype(np.float64)))]
        assert np.array_equal(ids[:n], want), (r, ids[:n], want)
        assert np.array_equal(ks[:n], row[want]), r          # (equal floats: the lists keep +0 for -0)
        assert not ids[n:].any() and not ks[n:].view(np.int32).any(), r
    return int(listed.sum())


def check_tile_lists(info, keys, V):
    """Each filtered row's tile list, against the tiles whose largest key
    (of the forward's own keys) reaches its last support key: equal when
    there are at most 31 of them, empty otherwise; and every support token
    lies in a listed tile."""
    T = keys.shape[0]
    ntv = -(-V // 256)
    pad = np.full((T, ntv * 256), -np.inf, np.float32)
    pad[:, :V] = keys
    tmax = pad.reshape(T, ntv, 256).max(2)
    for r in range(T):
        filt = (info["flags"][r] & binding.FLAG_FILTERED) != 0 and (info["flags"][r] & binding.FLAG_VALID) != 0
        if not filt:
            assert info["ntile"][r] == 0, r
            continue
        kthr = keys[r, info["id_thr"][r]]                        # the last support token's key
        want = np.nonzero(tmax[r] >= kthr)[0]
        got = info["tiles"][r, :info["ntile"][r]]
        if len(want) <= 31:
            assert np.array_equal(got, want), (r, got, want)
        else:
            assert info["ntile"][r] == 0, r


def check_recomputed_keys(rk, fk, info, g, y, V, dtype):
    """The backward's recomputed keys (NaN where it formed none) against the
    forward's, bit for bit: every row's keys, but a tiled row's only on its
    listed tiles (and none elsewhere) and none of a listed row's; the target
    key and the row maximum against the forward's state.  Returns (keys
    formed, tiled rows)."""
    rkc, fkc = np.asarray(rk), np.asarray(fk)
    T = fkc.shape[0]
    tiled = tiled_rows(info, g, V, dtype)
    listed = listed_rows(info, g, dtype)
    formed = np.ones((T, V), bool)
    formed[listed] = False
    for r in np.nonzero(tiled)[0]:
        formed[r] = False
        for j in info["tiles"][r, :info["ntile"][r]]:
            formed[r, 256 * j:256 * (j + 1)] = True
    assert np.array_equal(rkc[formed].view(np.int32), fkc[formed].view(np.int32)), \
        "recomputed keys differ from the forward's"
    assert np.isnan(rkc[~formed]).all()
    y = np.asarray(y)
    fy = formed[np.arange(T), y]
    assert fy[tiled].all()                                        # a tiled row's target lies in its tiles
    sy = rkc[np.arange(T), y]
    assert np.array_equal(sy[fy].view(np.int32), info["target_key"][fy].view(np.int32))
    mx = np.where(formed, rkc, -np.inf).max(1)
    assert np.array_equal(mx[~listed].view(np.int32), info["row_max"][~listed].view(np.int32))
    return int(formed.sum()), int(tiled.sum())
