"""GPU parity of the bf16 value lane, through the C ABI.

In the lane the projection's fp32 result is rounded to bf16, divided by the
row's temperature in fp32 and rounded to bf16 again; the support and the
log-sum-exps are taken on those keys and the selected logprob is rounded to
bf16.  The gradients treat both roundings as identity.

* The keys bit for bit: the lane's keys equal the oracle's rounding program
  applied to the GPU's own fp32 product (the fp32 lane's keys at T = 1), and
  match the oracle's keys from the exact product except where the fp32
  accumulation error moves a value across a bf16 rounding boundary (on a
  small fraction of the keys, by at most two bf16 ulps, one ulp of the
  rounded product scaled by the division, plus the accumulation error
  itself, which dominates where the product cancels).
* Against the oracle's lane on the GPU's keys: the support bit for bit, the
  logprob a bf16 value within max(2e-3, one bf16 ulp) (the two sides round
  nearly equal fp32 values), gradients within 1e-2 relative Frobenius error.
* The fused step in the lane: logprob and state bitwise equal to the unfused
  lane, gradients to the oracle's.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import GRAD_RTOL, check_support, dev, meta_of, rel_fro, say, targets, to_gpu
from sampling_transform_logprob_amd import binding, workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.load()


def _bf16_ulp(x):
    a = np.abs(np.asarray(x, np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.exp2(e - 7)


def _check_lane_logprob(lp, ref):
    lp = np.asarray(lp, np.float32)
    assert np.all((lp.view(np.uint32) & 0xFFFF) == 0), "logprob holds values that are not bf16"
    lp = lp.astype(np.float64)
    fin = np.isfinite(ref["logprob"])
    assert np.array_equal(np.isfinite(lp), fin)
    assert np.all(lp[~fin] == -np.inf)
    d = np.abs(lp[fin] - ref["logprob"][fin])
    tol = np.maximum(2e-3, _bf16_ulp(ref["logprob"][fin]) * 1.0001)
    assert np.all(d <= tol), f"logprob error {d.max()}"
    return float(d.max()) if d.size else 0.0, float((d > 0).mean()) if d.size else 0.0


def _case(name, T, V):
    w = workloads.make(name, T=T)
    if V is not None:
        w["W"] = w["W"][:V]
        w["V"] = V
        if not w["filtered"]:
            w["target_uniform"] = w["target_uniform"] % V
    return w


@pytest.mark.parametrize("name,T,V", [("headline", 200, 8192), ("ties", 160, 5000), ("identity", 160, 4000)])
def test_lane_keys_are_the_rounding_program_of_the_gpu_product(name, T, V):
    w = _case(name, T, V)
    G = to_gpu(w, np.zeros(T, np.int64))
    say(f"bf16 lane keys: {name} T={T} H={w['H']} V={V}")
    s = binding.scaled_logits(G["h"], G["W"], G["temperature"], lane="bf16").cpu().numpy()
    assert np.all((s.view(np.uint32) & 0xFFFF) == 0)
    z32 = binding.scaled_logits(G["h"], G["W"], None).cpu().numpy()       # the fp32 product
    own = oracle.bf16_lane_keys(z32.astype(np.float64), w["temperature"])
    assert np.array_equal(oracle.canonical_f32(s).view(np.uint32), own.view(np.uint32))
    exact = oracle.bf16_lane_keys(oracle.chunk_logits(w["h"], w["W"]), w["temperature"])
    diff = s != exact
    say(f"  keys differing from the exact product's program: {int(diff.sum())} of {s.size}")
    assert diff.mean() < 1e-3
    # bound: two bf16 ulps plus the fp32 accumulation error of the product
    # (relative to sum |h| |W| at most 1e-5), carried through the division
    scale = np.abs(w["h"]).astype(np.float64) @ np.abs(w["W"]).astype(np.float64).T
    acc = 1e-5 * scale / w["temperature"].astype(np.float64)[:, None]
    bound = 2.0001 * _bf16_ulp(exact) + 2 * acc
    assert np.all(np.abs(s[diff].astype(np.float64) - exact[diff]) <= bound[diff])


@pytest.mark.parametrize("name,T,V", [
    ("headline", 300, 8192),    # top-k 20 / top-p 0.8 at T = 0.7
    ("top_p", 260, 6000),       # V not a multiple of 64
    ("ties", 200, 5000),        # many equal bf16 keys
    ("identity", 200, 4000),    # unfiltered rows
])
def test_lane_matches_oracle(name, T, V):
    w = _case(name, T, V)
    y = np.asarray(targets(w), np.int64) % w["W"].shape[0]
    G = to_gpu(w, y)
    say(f"bf16 lane parity: {name} T={T} H={w['H']} V={V}")
    keys = binding.scaled_logits(G["h"], G["W"], G["temperature"], lane="bf16").cpu().numpy()
    lp, st = binding.forward(G["h"], G["W"], G["target"], **meta_of(G), lane="bf16", chunk_rows=128)
    ref = oracle.forward(w["h"], w["W"], y, w["temperature"], w["top_k"], w["top_p"], w["min_p"], keys=keys,
                         lane="bf16")
    info = binding.decode_state(st)
    near = check_support(info, ref, name)
    err, frac = _check_lane_logprob(lp.cpu().numpy(), ref)
    g = np.random.Generator(np.random.PCG64(9)).standard_normal(T)
    gg = torch.from_numpy(g.astype(np.float32)).to(dev())
    gh, gw = binding.backward(G["h"], G["W"], G["target"], st, gg, **meta_of(G), lane="bf16", vocab_slice=2048)
    dH, dW = oracle.backward(w["h"], w["W"], y, ref, g, w["temperature"])
    rh, rw = rel_fro(gh.float().cpu().numpy(), dH), rel_fro(gw.cpu().numpy(), dW)
    say(f"  near={near} logprob err={err:.2e} (rows off by one bf16 ulp: {frac:.3f}) dH rel={rh:.2e} "
        f"dW rel={rw:.2e} support sizes {info['n'].min()}..{info['n'].max()}")
    assert near == 0 and frac < 0.05 and rh < GRAD_RTOL and rw < GRAD_RTOL
    # the lane is not the fp32 program: its keys and logprobs differ
    lp32, _ = binding.forward(G["h"], G["W"], G["target"], **meta_of(G))
    assert not torch.equal(lp32, lp)


@pytest.mark.parametrize("name,T,V", [("headline", 300, 6000), ("ties", 200, 5000)])
def test_lane_fused_step(name, T, V):
    w = _case(name, T, V)
    y = np.asarray(targets(w), np.int64) % w["W"].shape[0]
    G = to_gpu(w, y)
    say(f"bf16 lane fused step: {name} T={T} V={V}")
    lp, st = binding.forward(G["h"], G["W"], G["target"], **meta_of(G), lane="bf16")
    rng = np.random.Generator(np.random.PCG64(21))
    A = torch.from_numpy(rng.uniform(-2, 2, T).astype(np.float32)).to(dev())
    old = torch.where(torch.isfinite(lp), lp, torch.full_like(lp, -5.0)) + 0.1
    f = binding.fused_policy_step(G["h"], G["W"], G["target"], A, old, **meta_of(G), objective="cispo",
                                  scale=1.0 / T, chunk_rows=128, lane="bf16")
    assert torch.equal(f["logprob"].view(torch.int32), lp.view(torch.int32)) and torch.equal(f["state"], st)
    keys = binding.scaled_logits(G["h"], G["W"], G["temperature"], lane="bf16").cpu().numpy()
    ref = oracle.forward(w["h"], w["W"], y, w["temperature"], w["top_k"], w["top_p"], w["min_p"], keys=keys,
                         lane="bf16")
    pg = oracle.policy_loss(ref["logprob"], A.cpu().numpy(), old.cpu().numpy(), "cispo", 0.2, 0.28, 1.0 / T)
    dH, dW = oracle.backward(w["h"], w["W"], y, ref, pg["g"], w["temperature"])
    rh = rel_fro(f["grad_hidden"].float().cpu().numpy(), dH)
    rw = rel_fro(f["grad_weight"].cpu().numpy(), dW)
    say(f"  bitwise logprob/state vs the unfused lane; dH rel={rh:.2e} dW rel={rw:.2e}")
    assert rh < GRAD_RTOL and rw < GRAD_RTOL
