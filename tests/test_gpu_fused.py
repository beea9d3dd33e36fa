"""GPU parity of the fused head + policy-gradient step, through the C ABI.
The step forms dlogits from keys the forward's sweep keeps.  With row
classes (bf16 operands with a filter given, or the fp8 lane) the sweep keeps
each small support with its keys in the state and the step is the forward,
the loss and the classed backward in one call; dense (fp32, or bf16 with no
filter) it forms every row's dz from the chunk's keys and needs no recompute
product at all.

* Against the oracle (forward, token loss and VJP in fp64) at the core's
  bar: logprob within 2e-3, the summed loss within 1e-3 relative, and
  gradients within 1e-2 relative Frobenius error.  Several chunks are used,
  with a ragged last one.
* Against the unfused sequence (stce_forward, stce_policy_loss,
  stce_backward) on the same inputs:
  - logprob, state, loss and ratio are bitwise equal, since the same kernels
    decide them;
  - gradients are equal up to fp32 summation order: dz is bitwise the
    recompute's, but the products reduce in another order;
  - inactive, invalid and out-of-support rows, a frozen head, weight-gradient
    accumulation and the side outputs are all covered.
* With row classes every output equals the unfused sequence's bit for bit,
  on batches that mix every class within a chunk (listed, tiled, sparse,
  dense, no gradient), on the fp8 lane, for a frozen head and with
  weight-gradient accumulation.
* The dense path, taken by bf16 problems with no filter arrays, against the
  oracle and against the unfused sequence.
* At the full headline size, in the default schedule, the same comparison
  with the unfused path.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import GRAD_RTOL, check_logprob, dev, meta_of, rel_fro, say, targets, to_gpu
from sampling_transform_logprob_amd import binding, workloads

pytestmark = pytest.mark.gpu

EL, EH = 0.2, 0.28


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.load()


def _pg_inputs(lp, seed):
    """Advantages and behaviour logprobs putting the ratios on both sides of
    both clip bounds (fp32, seeded)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    T = lp.shape[0]
    A = rng.choice([-1.0, 1.0], T) * rng.uniform(0.1, 3.0, T)
    off = rng.choice([-1.2, -0.4, -0.05, 0.0, 0.1, 0.5, 1.4], T) + rng.uniform(-0.02, 0.02, T)
    finite = np.where(np.isfinite(lp), lp, -5.0)
    return A.astype(np.float32), (finite + off).astype(np.float32)


def _bits(t):
    return t.contiguous().view(torch.int32) if t.dtype == torch.float32 else t


def _same(a, b):
    return torch.equal(_bits(a), _bits(b))


def _setup(name, T, V):
    w = workloads.make(name, T=T)
    if V is not None:
        w["W"] = w["W"][:V]
        w["V"] = V
    y = np.asarray(targets(w), np.int64) % w["W"].shape[0]
    return w, y, to_gpu(w, y)


@pytest.mark.parametrize("name,T,V,objective,chunk", [
    ("headline", 200, 4096, "cispo", 64),    # 4 chunks, the last of 8 rows
    ("top_p", 130, 6000, "clip", 64),        # V not a multiple of 64
    ("tiny", 64, None, "clip", 0),           # fp32 operands, one chunk
    ("identity", 100, 3000, "cispo", 64),    # unfiltered rows
])
def test_fused_step_matches_oracle(name, T, V, objective, chunk):
    w, y, G = _setup(name, T, V)
    V = w["W"].shape[0]
    say(f"fused step vs oracle: {name} T={T} H={w['H']} V={V} {objective} chunk={chunk}")
    keys = binding.scaled_logits(G["h"], G["W"], G["temperature"]).cpu().numpy()
    ref = oracle.forward(w["h"], w["W"], y, w["temperature"], w["top_k"], w["top_p"], w["min_p"], keys=keys)
    A, old = _pg_inputs(ref["logprob"], 11)
    sc = 1.0 / T
    out = binding.fused_policy_step(G["h"], G["W"], G["target"], torch.from_numpy(A).to(dev()),
                                    torch.from_numpy(old).to(dev()), **meta_of(G), objective=objective,
                                    eps_low=EL, eps_high=EH, scale=sc, chunk_rows=chunk)
    err = check_logprob(out["logprob"].cpu().numpy(), ref)
    pg = oracle.policy_loss(ref["logprob"], A, old, objective, EL, EH, sc)
    dH, dW = oracle.backward(w["h"], w["W"], y, ref, pg["g"], w["temperature"])
    rl = abs(float(out["loss"].double().sum()) - pg["loss"].sum()) / max(1e-12, abs(pg["loss"]).sum())
    rh = rel_fro(out["grad_hidden"].float().cpu().numpy(), dH)
    rw = rel_fro(out["grad_weight"].cpu().numpy(), dW)
    say(f"  logprob err {err:.2e}  loss rel {rl:.2e}  dH rel {rh:.2e}  dW rel {rw:.2e}")
    assert rl < 1e-3 and rh < GRAD_RTOL and rw < GRAD_RTOL


def _unfused(G, A, old, objective, sc, ignore_index=None, side=False, gw0=None, meta=None, need_weight=True,
             recompute_all=False):
    meta = meta_of(G) if meta is None else meta
    ws = G.get("weight_scale")
    r = binding.forward(G["h"], G["W"], G["target"], **meta, check=False, side=side,
                        ignore_index=ignore_index, weight_scale=ws)
    lp, st = r[0], r[1]
    loss, g, ratio = binding.policy_loss(lp, A, old, objective, EL, EH, sc, st)
    gw = None if gw0 is None else gw0.clone()
    gh, gw = binding.backward(G["h"], G["W"], G["target"], st, g, **meta, grad_weight=gw,
                              accumulate_grad_weight=gw0 is not None, ignore_index=ignore_index,
                              weight_scale=ws, need_weight=need_weight, recompute_all=recompute_all)
    out = dict(logprob=lp, state=st, loss=loss, ratio=ratio, grad_hidden=gh, grad_weight=gw)
    if side:
        out.update(r[2])
    return out


@pytest.mark.parametrize("name,T,V", [("headline", 300, 5000), ("tiny", 64, None)])
def test_fused_step_equals_unfused_sequence(name, T, V):
    w, y, G = _setup(name, T, V)
    V = w["W"].shape[0]
    IGN = -100
    # special rows: out of support (-inf), invalid metadata (NaN), inactive
    low = int(np.argsort(w["W"].astype(np.float64) @ w["h"][3].astype(np.float64))[0])
    G["top_k"][3] = 3
    G["target"][3] = low
    G["top_p"][7] = 1.5
    G["target"][10:13] = IGN
    lp0, _ = binding.forward(G["h"], G["W"], G["target"], **meta_of(G), check=False, ignore_index=IGN)
    A, old = _pg_inputs(lp0.cpu().numpy(), 13)
    A, old = torch.from_numpy(A).to(dev()), torch.from_numpy(old).to(dev())
    sc = 1.0 / T
    say(f"fused vs unfused: {name} T={T} H={w['H']} V={V}")
    u = _unfused(G, A, old, "cispo", sc, ignore_index=IGN, side=True)
    prob64, _ = binding.make_problem(G["h"], G["W"], G["target"], chunk_rows=64)
    full64, min64 = binding.fused_workspace_bytes(prob64)
    two = (min64 + (full64 - min64) // (-(-T // 64) - 1)) if full64 > min64 else None
    # 64-row chunks, all in one weight-gradient group; 64-row chunks two to a
    # group (a workspace with room for two chunks' vocab-major dz), the last
    # group partial; the default chunk
    for chunk, nbytes in ((64, None), (64, two), (0, None)):
        ws = None if nbytes is None else torch.empty(nbytes, dtype=torch.uint8, device=dev())
        f = binding.fused_policy_step(G["h"], G["W"], G["target"], A, old, **meta_of(G), objective="cispo",
                                      eps_low=EL, eps_high=EH, scale=sc, chunk_rows=chunk, side=True,
                                      ignore_index=IGN, check=False, workspace=ws)
        if not _same(f["state"], u["state"]):
            df, du = binding.decode_state(f["state"]), binding.decode_state(u["state"])
            diff = {k: np.nonzero(df[k].view(np.uint32) != du[k].view(np.uint32))[0][:8].tolist() for k in df}
            raise AssertionError(f"chunk {chunk}: state differs (field: rows) {diff}")
        for k in ("logprob", "loss", "ratio", "lse_full", "entropy_full", "entropy_support"):
            assert _same(f[k], u[k]), (chunk, k)
        lpc = f["logprob"].cpu().numpy()
        assert lpc[3] == -np.inf and np.isnan(lpc[7]) and np.all(lpc[10:13] == 0.0)
        ghf = f["grad_hidden"].float()
        assert torch.count_nonzero(ghf[[3, 7, 10, 11, 12]]) == 0
        rh = rel_fro(ghf.cpu().numpy(), u["grad_hidden"].float().cpu().numpy())
        rw = rel_fro(f["grad_weight"].cpu().numpy(), u["grad_weight"].cpu().numpy())
        say(f"  chunk {chunk or 'default'}{'' if nbytes is None else ', two chunks a group'}: bitwise "
            f"logprob/state/loss/ratio/side; dH rel {rh:.2e}  dW rel {rw:.2e}")
        assert rh < 1e-3 and rw < 1e-5
    # frozen head: the same hidden gradient, no weight gradient
    fz = binding.fused_policy_step(G["h"], G["W"], G["target"], A, old, **meta_of(G), objective="cispo",
                                   eps_low=EL, eps_high=EH, scale=sc, chunk_rows=0, need_weight=False,
                                   ignore_index=IGN, check=False)
    assert fz["grad_weight"] is None and _same(fz["grad_hidden"], f["grad_hidden"])
    # loss only
    lo = binding.fused_policy_step(G["h"], G["W"], G["target"], A, old, **meta_of(G), objective="clip",
                                   eps_low=EL, eps_high=EH, scale=sc, need_hidden=False, need_weight=False,
                                   ignore_index=IGN, check=False)
    uc = _unfused(G, A, old, "clip", sc, ignore_index=IGN)
    assert _same(lo["loss"], uc["loss"]) and lo["grad_hidden"] is None
    # weight-gradient accumulation onto an existing gradient
    gw0 = torch.randn(V, w["H"], device=dev(), dtype=torch.float32)
    ua = _unfused(G, A, old, "clip", sc, ignore_index=IGN, gw0=gw0)
    fa = binding.fused_policy_step(G["h"], G["W"], G["target"], A, old, **meta_of(G), objective="clip",
                                   eps_low=EL, eps_high=EH, scale=sc, chunk_rows=64, grad_weight=gw0.clone(),
                                   accumulate_grad_weight=True, ignore_index=IGN, check=False)
    d_f, d_u = (fa["grad_weight"] - gw0).cpu().numpy(), (ua["grad_weight"] - gw0).cpu().numpy()
    ra = rel_fro(d_f, d_u)
    say(f"  accumulate: dW increment rel {ra:.2e}")
    assert ra < 1e-4


def test_full_size_headline_fused_equals_unfused():
    w = workloads.make("headline")
    T, H, V = w["T"], w["H"], w["V"]
    say(f"full size fused step: T={T} H={H} V={V}")
    y = w["target_uniform"].copy()
    G0 = to_gpu(w, y)
    am = torch.cat([(G0["h"][r:r + 2048].float() @ G0["W"].float().T).argmax(1)
                    for r in range(0, T, 2048)]).cpu().numpy()
    del G0
    y = np.where(np.arange(T) % 10 == 0, y, am)
    G = to_gpu(w, y)
    lp0, _ = binding.forward(G["h"], G["W"], G["target"], **meta_of(G))
    A, old = _pg_inputs(lp0.cpu().numpy(), 17)
    A, old = torch.from_numpy(A).to(dev()), torch.from_numpy(old).to(dev())
    u = _unfused(G, A, old, "cispo", 1.0 / T)
    torch.cuda.synchronize()
    say("  unfused done")
    f = binding.fused_policy_step(G["h"], G["W"], G["target"], A, old, **meta_of(G), objective="cispo",
                                  eps_low=EL, eps_high=EH, scale=1.0 / T)
    torch.cuda.synchronize()
    for k in ("logprob", "state", "loss", "ratio"):
        assert _same(f[k], u[k]), k
    gh_f, gh_u = f["grad_hidden"].float(), u["grad_hidden"].float()
    rh = ((gh_f - gh_u).norm() / gh_u.norm()).item()
    rw = ((f["grad_weight"] - u["grad_weight"]).norm() / u["grad_weight"].norm()).item()
    say(f"  bitwise logprob/state/loss/ratio; dH rel {rh:.2e}  dW rel {rw:.2e}  "
        f"-inf rows {int(torch.isinf(f['logprob']).sum())}")
    assert rh < 1e-3 and rw < 1e-4


def test_many_chunks_equal_the_unfused_sequence():
    """18 chunks of 64 rows: the selection of every chunk overlaps the next
    projection on the side stream, whose events are reused chunk after
    chunk; logprob, state and loss stay bitwise those of the unfused path."""
    w, y, G = _setup("top_p", 1100, 3000)
    lp0, _ = binding.forward(G["h"], G["W"], G["target"], **meta_of(G), check=False)
    A, old = _pg_inputs(lp0.cpu().numpy(), 19)
    A, old = torch.from_numpy(A).to(dev()), torch.from_numpy(old).to(dev())
    say("fused vs unfused: top_p T=1100 V=3000, 18 chunks")
    u = _unfused(G, A, old, "clip", 1.0 / 1100)
    f = binding.fused_policy_step(G["h"], G["W"], G["target"], A, old, **meta_of(G), objective="clip",
                                  eps_low=EL, eps_high=EH, scale=1.0 / 1100, chunk_rows=64, check=False)
    for k in ("logprob", "state", "loss", "ratio"):
        assert _same(f[k], u[k]), k
    rh = rel_fro(f["grad_hidden"].float().cpu().numpy(), u["grad_hidden"].float().cpu().numpy())
    rw = rel_fro(f["grad_weight"].cpu().numpy(), u["grad_weight"].cpu().numpy())
    say(f"  bitwise logprob/state/loss/ratio; dH rel {rh:.2e}  dW rel {rw:.2e}")
    assert rh < 1e-3 and rw < 1e-5


def _classed_case(name, T, V):
    """A small batch of the named workload whose chunks mix every row class:
    every fifth row unfiltered (its support the whole vocabulary: dense),
    every seventh a top-p row of a wide support (over 128 tokens: dense),
    every eleventh a top-64 row, every thirteenth a top-120 row (more tokens
    than the vocabulary has tiles, so decided from a histogram), the rest
    top-k rows; one row's target outside its support, one invalid row.  The
    small supports are listed in the state; with every row recomputed they
    are tiled, or sparse past 31 tiles."""
    w = workloads.make(name, T=T)
    if V is not None and V < w["V"]:
        w["W"], w["V"] = w["W"][:V], V
        if w.get("w_scale") is not None:
            w["w_scale"] = w["w_scale"][:V]
        w["target_uniform"] = w["target_uniform"] % V
    w["top_k"][::5], w["top_p"][::5], w["min_p"][::5] = 0, 1.0, 0.0
    w["top_k"][3::7], w["top_p"][3::7] = 0, 0.9
    w["top_k"][6::11] = 64
    w["top_k"][9::13], w["top_p"][9::13], w["min_p"][9::13] = 120, 1.0, 0.0
    y = np.asarray(targets(w), np.int64) % w["W"].shape[0]
    G = to_gpu(w, y)
    # row 1: top-2 with the target at the lowest logit (the oracle's)
    if w["dtype"] == "fp8":
        z1 = oracle.fp8_logits(w["h"][1:2], w["W"], w["w_scale"])[0]
    else:
        z1 = w["W"].astype(np.float64) @ w["h"][1].astype(np.float64)
    G["top_k"][1], G["top_p"][1] = 2, 1.0
    G["target"][1] = int(np.argmin(z1))
    G["top_p"][2] = 1.5                                   # invalid metadata
    return w, y, G


@pytest.mark.parametrize("name,T,V,chunk", [
    ("headline", 300, 5000, 64),      # 5 chunks, the last of 44 rows
    ("headline", 200, 6000, 0),       # one chunk (V above the selection's whole-row window of 3712 tokens)
    ("top_p", 260, 6000, 128),
    ("headline_fp8", 300, 30000, 128),
])
def test_classed_fused_step_equals_the_unfused_sequence_bitwise(name, T, V, chunk):
    w, y, G = _classed_case(name, T, V)
    V = w["W"].shape[0]
    ws = G.get("weight_scale")
    lp0, st0 = binding.forward(G["h"], G["W"], G["target"], **meta_of(G), check=False, weight_scale=ws)
    A, old = _pg_inputs(lp0.cpu().numpy(), 23)
    A, old = torch.from_numpy(A).to(dev()), torch.from_numpy(old).to(dev())
    sc = 1.0 / T
    u = _unfused(G, A, old, "clip", sc)
    full, least = binding.fused_workspace_bytes(binding.make_problem(G["h"], G["W"], G["target"], **meta_of(G),
                                                                     weight_scale=ws)[0])
    assert full == least                                  # the classed path's workspace has no groups
    f = binding.fused_policy_step(G["h"], G["W"], G["target"], A, old, **meta_of(G), objective="clip",
                                  eps_low=EL, eps_high=EH, scale=sc, chunk_rows=chunk, check=False,
                                  weight_scale=ws)
    info = binding.decode_state(f["state"])
    fl = info["flags"]
    live = ((fl & binding.FLAG_VALID) != 0) & ((fl & binding.FLAG_IN_SUPPORT) != 0)
    filt = live & ((fl & binding.FLAG_FILTERED) != 0)
    small = filt & (info["n"] <= 128)
    listed = small & ((fl & binding.FLAG_LISTED) != 0)
    tiled = small & (info["ntile"] > 0)                  # (with every row recomputed)
    sparse = small & (info["ntile"] == 0)
    say(f"classed fused vs unfused: {name} T={T} V={V} chunk={chunk or 'default'}: rows dense "
        f"{int((live & ~filt).sum() + (filt & (info['n'] > 128)).sum())}, listed {int(listed.sum())}, tiled "
        f"{int(tiled.sum())}, sparse {int(sparse.sum())}, no gradient {int((~live).sum())}")
    assert np.array_equal(listed, small)                  # every small support is listed
    assert listed.sum() > 0 and (live & ~filt).sum() > 0 and (~live).sum() >= 2
    for k in ("logprob", "state", "loss", "ratio", "grad_hidden", "grad_weight"):
        assert _same(f[k], u[k]), k
    # every row recomputed (tile or whole-vocabulary recompute) in both
    fr = binding.fused_policy_step(G["h"], G["W"], G["target"], A, old, **meta_of(G), objective="clip",
                                   eps_low=EL, eps_high=EH, scale=sc, chunk_rows=chunk, check=False,
                                   weight_scale=ws, recompute_all=True)
    ur = _unfused(G, A, old, "clip", sc, recompute_all=True)
    for k in ("grad_hidden", "grad_weight"):
        assert _same(fr[k], ur[k]), k
    assert _same(fr["grad_hidden"], u["grad_hidden"])    # a row's dH sums its entries in vocabulary order
    # a frozen head: the same hidden gradient; weight-gradient accumulation:
    # the same sum onto the same start
    fz = binding.fused_policy_step(G["h"], G["W"], G["target"], A, old, **meta_of(G), objective="clip",
                                   eps_low=EL, eps_high=EH, scale=sc, chunk_rows=chunk, need_weight=False,
                                   check=False, weight_scale=ws)
    assert fz["grad_weight"] is None and _same(fz["grad_hidden"], u["grad_hidden"])
    gw0 = torch.randn(V, w["H"], device=dev(), dtype=torch.float32)
    ua = _unfused(G, A, old, "clip", sc, gw0=gw0)
    fa = binding.fused_policy_step(G["h"], G["W"], G["target"], A, old, **meta_of(G), objective="clip",
                                   eps_low=EL, eps_high=EH, scale=sc, chunk_rows=chunk, grad_weight=gw0.clone(),
                                   accumulate_grad_weight=True, check=False, weight_scale=ws)
    assert _same(fa["grad_weight"], ua["grad_weight"])
    say("  bitwise: logprob, state, loss, ratio, grad_hidden, grad_weight; frozen head; accumulation")


def test_classed_fused_step_matches_the_oracle_on_the_fp8_lane():
    w, y, G = _classed_case("headline_fp8", 160, 20000)
    G["top_p"][2] = float(w["top_p"][2])                 # (the oracle takes valid metadata only)
    V = w["W"].shape[0]
    ws = G["weight_scale"]
    say(f"classed fused step vs oracle, fp8 lane: T=160 H={w['H']} V={V}")
    keys = binding.scaled_logits(G["h"], G["W"], G["temperature"], weight_scale=ws).cpu().numpy()
    meta = {k: G[k].cpu().numpy() for k in ("top_k", "top_p", "min_p")}
    yy = G["target"].cpu().numpy()
    ref = oracle.forward(w["h"], w["W"], yy, w["temperature"], meta["top_k"], meta["top_p"], meta["min_p"],
                         keys=keys, lane="fp8", w_scale=w["w_scale"])
    A, old = _pg_inputs(ref["logprob"], 29)
    sc = 1.0 / 160
    out = binding.fused_policy_step(G["h"], G["W"], G["target"], torch.from_numpy(A).to(dev()),
                                    torch.from_numpy(old).to(dev()), **meta_of(G), objective="cispo",
                                    eps_low=EL, eps_high=EH, scale=sc, chunk_rows=64, check=False, weight_scale=ws)
    fin = np.isfinite(ref["logprob"])
    lp = out["logprob"].cpu().numpy()
    assert np.array_equal(np.isfinite(lp), fin)
    err = float(np.abs(lp[fin] - ref["logprob"][fin]).max())
    pg = oracle.policy_loss(ref["logprob"], A, old, "cispo", EL, EH, sc)
    dH, dW = oracle.backward(w["h"], w["W"], yy, ref, pg["g"], w["temperature"], w_scale=w["w_scale"])
    rh = rel_fro(out["grad_hidden"].float().cpu().numpy(), dH)
    rw = rel_fro(out["grad_weight"].cpu().numpy(), dW)
    say(f"  logprob err {err:.2e}  dH rel {rh:.2e}  dW rel {rw:.2e}")
    assert err < 2e-3 and rh < GRAD_RTOL and rw < GRAD_RTOL


def test_dense_fused_path_without_filters():
    """bf16 with no filter arrays: every row's support is the vocabulary, the
    step takes its dense path (dz of every row, two gradient products),
    against the oracle and the unfused sequence."""
    w, y, G = _setup("headline", 200, 4096)
    V = w["W"].shape[0]
    T = 200
    y = np.asarray(w["target_uniform"], np.int64) % V
    G["target"] = torch.from_numpy(y).to(dev())
    none = dict(temperature=G["temperature"], top_k=None, top_p=None, min_p=None)
    prob, _ = binding.make_problem(G["h"], G["W"], G["target"], **none, chunk_rows=64)
    full, least = binding.fused_workspace_bytes(prob)
    assert full > least                                   # the dense path's grouped workspace
    say(f"dense fused path (no filters): headline T={T} V={V}")
    keys = binding.scaled_logits(G["h"], G["W"], G["temperature"]).cpu().numpy()
    zk, op, zm = np.zeros(T, np.int32), np.ones(T, np.float32), np.zeros(T, np.float32)
    ref = oracle.forward(w["h"], w["W"], y, w["temperature"], zk, op, zm, keys=keys)
    A, old = _pg_inputs(ref["logprob"], 31)
    A, old = torch.from_numpy(A).to(dev()), torch.from_numpy(old).to(dev())
    sc = 1.0 / T
    f = binding.fused_policy_step(G["h"], G["W"], G["target"], A, old, **none, objective="cispo", eps_low=EL,
                                  eps_high=EH, scale=sc, chunk_rows=64)
    u = _unfused(G, A, old, "cispo", sc, meta=none)
    for k in ("logprob", "state", "loss", "ratio"):
        assert _same(f[k], u[k]), k
    pg = oracle.policy_loss(ref["logprob"], A.cpu().numpy(), old.cpu().numpy(), "cispo", EL, EH, sc)
    dH, dW = oracle.backward(w["h"], w["W"], y, ref, pg["g"], w["temperature"])
    rh = rel_fro(f["grad_hidden"].float().cpu().numpy(), dH)
    rw = rel_fro(f["grad_weight"].cpu().numpy(), dW)
    ruh = rel_fro(f["grad_hidden"].float().cpu().numpy(), u["grad_hidden"].float().cpu().numpy())
    ruw = rel_fro(f["grad_weight"].cpu().numpy(), u["grad_weight"].cpu().numpy())
    say(f"  vs oracle: dH rel {rh:.2e}  dW rel {rw:.2e}; vs unfused: dH rel {ruh:.2e}  dW rel {ruw:.2e}")
    assert rh < GRAD_RTOL and rw < GRAD_RTOL and ruh < 1e-3 and ruw < 1e-5
