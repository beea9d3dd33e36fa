"""GPU parity of the scalar pre-GEMM temperature convention, through the C ABI.

With one scalar temperature Ts for the lane, the library divides the hidden
states before the projection (h' = h / Ts in fp32, rounded to the operand
dtype) and scores s = fl32(h' W^T); the gradients are those of that s
(dW = dz^T h', dH = (dz W) / Ts with dz = g (1[j == y] - q)).

* h' itself, bit for bit against the oracle's rounding: with W the identity
  (V = H) every key is one exact product, so the keys are h'.
* Against the oracle at a generic Ts (0.7): the support bit for bit on the
  GPU's own keys, logprob within 2e-3, gradients within 1e-2 relative
  Frobenius error; forward, backward, and the fused step.
* Ts = 0.5 divides exactly, so the convention must reproduce the per-row
  post-GEMM convention with every row at 0.5 bit for bit: logprob, state,
  both gradients, and the fused step's outputs.  Ts = 1 must reproduce the
  run without temperature.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import GRAD_RTOL, check_logprob, check_support, dev, rel_fro, say
from sampling_transform_logprob_amd import binding, workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.load()


def _case(name, T, V):
    w = workloads.make(name, T=T)
    if V is not None:
        w["W"] = w["W"][:V]
        w["V"] = V
    return w


def _gpu_meta(w):
    d = dev()
    return dict(top_k=torch.from_numpy(w["top_k"]).to(d), top_p=torch.from_numpy(w["top_p"]).to(d),
                min_p=torch.from_numpy(w["min_p"]).to(d))


def _operands(w):
    dt = torch.float32 if w["dtype"] == "f32" else torch.bfloat16
    return (torch.from_numpy(w["h"]).to(dev()).to(dt), torch.from_numpy(w["W"]).to(dev()).to(dt))


def _bits(t):
    return t.contiguous().view(torch.int32) if t.dtype == torch.float32 else t


def _same(a, b):
    return torch.equal(_bits(a), _bits(b))


@pytest.mark.parametrize("dtype,ts", [("bf16", 0.7), ("bf16", 3.1), ("f32", 0.7), ("bf16", 0.013)])
def test_scaled_hidden_is_the_oracles_bit_for_bit(dtype, ts):
    rng = np.random.Generator(np.random.PCG64(5))
    T, H = 96, 136
    h = (rng.standard_normal((T, H)) * np.exp(rng.uniform(-4, 4, (T, 1)))).astype(np.float32)
    if dtype == "bf16":
        h = oracle.round_to_bf16(h)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    hg = torch.from_numpy(h).to(dev()).to(tdt)
    eye = torch.eye(H, dtype=tdt, device=dev())
    say(f"scaled hidden through an identity head: {dtype} Ts={ts} T={T} H={H}")
    keys = binding.scaled_logits(hg, eye, pre_gemm_temperature=ts).cpu().numpy()
    ref = oracle.pre_gemm_hidden(h, ts, dtype)
    assert np.array_equal(keys.view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("name,T,V,ts", [
    ("headline", 300, 8192, 0.7),   # bf16, top-k / top-p
    ("top_p", 260, 6000, 1.3),      # V not a multiple of 64
    ("ties", 200, 5000, 0.7),       # tied keys
    ("tiny", 64, None, 0.7),        # fp32 operands
])
def test_pre_gemm_temperature_matches_oracle(name, T, V, ts):
    w = _case(name, T, V)
    V = w["W"].shape[0]
    op = "f32" if w["dtype"] == "f32" else "bf16"
    hs = oracle.pre_gemm_hidden(w["h"], ts, op)
    y = (oracle.sample_targets(hs, w["W"], None, w["top_k"], w["top_p"], w["min_p"], w["u"])
         if w["filtered"] else w["target_uniform"] % V)
    y[::17] = (y[::17] + 7) % V                              # some targets outside the support
    h, W = _operands(w)
    meta = _gpu_meta(w)
    tgt = torch.from_numpy(np.asarray(y, np.int64)).to(dev())
    say(f"pre-GEMM parity {name}: T={T} H={w['H']} V={V} Ts={ts}")
    keys = binding.scaled_logits(h, W, pre_gemm_temperature=ts).cpu().numpy()
    z64 = oracle.chunk_logits(hs, w["W"])
    scale = np.abs(hs).astype(np.float64) @ np.abs(w["W"]).astype(np.float64).T
    assert (np.abs(keys - z64) / scale).max() < 1e-5         # fp32 accumulation of exact products of h'
    lp, st = binding.forward(h, W, tgt, **meta, pre_gemm_temperature=ts, chunk_rows=128)
    ref = oracle.forward(hs, w["W"], y, None, w["top_k"], w["top_p"], w["min_p"], keys=keys)
    info = binding.decode_state(st)
    near = check_support(info, ref, name)
    err = check_logprob(lp.cpu().numpy(), ref)
    g = np.random.Generator(np.random.PCG64(3)).standard_normal(T)
    gg = torch.from_numpy(g.astype(np.float32)).to(dev())
    gh, gw = binding.backward(h, W, tgt, st, gg, **meta, pre_gemm_temperature=ts, vocab_slice=2048)
    dH, dW = oracle.backward_pre_gemm(hs, w["W"], y, ref, g, ts)
    rh, rw = rel_fro(gh.float().cpu().numpy(), dH), rel_fro(gw.cpu().numpy(), dW)
    say(f"  near={near} logprob err={err:.2e} dH rel={rh:.2e} dW rel={rw:.2e} "
        f"-inf rows {int(np.isinf(lp.cpu().numpy()).sum())}")
    assert near == 0 and rh < GRAD_RTOL and rw < GRAD_RTOL
    # the fused step on the same problem: the same forward bits, the
    # oracle's gradients of sum(loss)
    A = np.random.Generator(np.random.PCG64(4)).uniform(-2, 2, T).astype(np.float32)
    old = np.where(np.isfinite(ref["logprob"]), ref["logprob"], -5.0).astype(np.float32) + 0.05
    f = binding.fused_policy_step(h, W, tgt, torch.from_numpy(A).to(dev()), torch.from_numpy(old).to(dev()), **meta,
                                  objective="cispo", scale=1.0 / T, chunk_rows=128, pre_gemm_temperature=ts)
    assert _same(f["logprob"], lp) and _same(f["state"], st)
    pg = oracle.policy_loss(ref["logprob"], A, old, "cispo", 0.2, 0.28, 1.0 / T)
    fH, fW = oracle.backward_pre_gemm(hs, w["W"], y, ref, pg["g"], ts)
    rfh = rel_fro(f["grad_hidden"].float().cpu().numpy(), fH)
    rfw = rel_fro(f["grad_weight"].cpu().numpy(), fW)
    say(f"  fused step: dH rel={rfh:.2e} dW rel={rfw:.2e}")
    assert rfh < GRAD_RTOL and rfw < GRAD_RTOL


@pytest.mark.parametrize("name,T,V", [("headline", 300, 6000), ("tiny", 64, None)])
def test_power_of_two_temperature_reproduces_the_per_row_convention(name, T, V):
    w = _case(name, T, V)
    V = w["W"].shape[0]
    h, W = _operands(w)
    meta = _gpu_meta(w)
    y = np.where(np.arange(T) % 5 == 0, w["target_uniform"] % V,
                 (w["h"].astype(np.float64) @ w["W"].astype(np.float64).T).argmax(1))
    tgt = torch.from_numpy(np.asarray(y, np.int64)).to(dev())
    half = torch.full((T,), 0.5, dtype=torch.float32, device=dev())
    say(f"Ts = 0.5 against a per-row 0.5: {name} T={T} V={V}")
    assert _same(binding.scaled_logits(h, W, pre_gemm_temperature=0.5), binding.scaled_logits(h, W, half))
    lp1, st1 = binding.forward(h, W, tgt, half, **meta)
    lp2, st2 = binding.forward(h, W, tgt, **meta, pre_gemm_temperature=0.5)
    assert _same(lp1, lp2) and _same(st1, st2)
    g = torch.randn(T, device=dev())
    a = binding.backward(h, W, tgt, st1, g, half, **meta)
    b = binding.backward(h, W, tgt, st2, g, **meta, pre_gemm_temperature=0.5)
    assert _same(a[0], b[0]) and _same(a[1], b[1])
    A = torch.randn(T, device=dev())
    old = torch.where(torch.isfinite(lp1), lp1, torch.full_like(lp1, -5.0)) + 0.1
    kw = dict(objective="clip", scale=1.0 / T, chunk_rows=128)
    f1 = binding.fused_policy_step(h, W, tgt, A, old, half, **meta, **kw)
    f2 = binding.fused_policy_step(h, W, tgt, A, old, **meta, **kw, pre_gemm_temperature=0.5)
    for k in ("logprob", "state", "loss", "ratio", "grad_hidden", "grad_weight"):
        assert _same(f1[k], f2[k]), k
    # Ts = 1: the run without temperature
    lp0, st0 = binding.forward(h, W, tgt, **meta)
    lp3, st3 = binding.forward(h, W, tgt, **meta, pre_gemm_temperature=1.0)
    assert _same(lp0, lp3) and _same(st0, st3)
    c = binding.backward(h, W, tgt, st0, g, **meta)
    d = binding.backward(h, W, tgt, st3, g, **meta, pre_gemm_temperature=1.0)
    assert _same(c[0], d[0]) and _same(c[1], d[1])
    say(f"  bitwise: keys, logprob, state, grads, fused step; -inf rows {int(torch.isinf(lp1).sum())}")
