"""GPU parity of the policy-gradient token loss (CISPO and the clipped
surrogate) on the selected logprob, through the C ABI, against the oracle.

* The per-row kernel is compared with ``oracle.policy_loss`` on the same fp32
  inputs (the GPU's logprobs): fp32 arithmetic against fp64, so losses and
  gradients agree to 1e-5 relative (expf and a few products); ratios of
  -inf rows, NaN rows and every clip branch are covered.
* The fused step (forward, loss, backward with the loss's upstream
  gradient) is compared end to end with the oracle's forward, loss and VJP
  at the core's bar: gradients within 1e-2 relative Frobenius error.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import GRAD_RTOL, dev, meta_of, rel_fro, say, targets, to_gpu
from sampling_transform_logprob_amd import binding, workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.load()


def _pg_inputs(lp, seed):
    """Advantages and behaviour logprobs that put the ratios on both sides of
    both clip bounds (fp32 values, seeded)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    T = lp.shape[0]
    A = rng.choice([-1.0, 1.0], T) * rng.uniform(0.1, 3.0, T)
    off = rng.choice([-1.2, -0.4, -0.05, 0.0, 0.1, 0.5, 1.4], T) + rng.uniform(-0.02, 0.02, T)
    finite = np.where(np.isfinite(lp), lp, -5.0)
    return A.astype(np.float32), (finite + off).astype(np.float32)


@pytest.mark.parametrize("objective", ["cispo", "clip"])
def test_policy_loss_kernel_matches_oracle(objective):
    w = workloads.make("tiny", T=64)
    y = targets(w)
    y[5] = int(np.argsort(w["W"] @ w["h"][5])[0])      # lowest logit: outside the top-3 support set below
    G = to_gpu(w, y)
    G["top_k"][5] = 3                                   # row 5: top-3 support, target outside it
    G["top_p"][9] = 1.5                                 # row 9: invalid metadata -> NaN logprob
    lp, st = binding.forward(G["h"], G["W"], G["target"], **meta_of(G), check=False)
    lpc = lp.cpu().numpy()
    assert lpc[5] == -np.inf and np.isnan(lpc[9])
    A, old = _pg_inputs(lpc, 5)
    say(f"policy loss kernel: {objective}, T=64")
    el, eh, sc = 0.2, 0.28, 1.0 / 48
    loss, g, ratio = binding.policy_loss(lp, torch.from_numpy(A).to(dev()), torch.from_numpy(old).to(dev()),
                                         objective, el, eh, sc)
    ref = oracle.policy_loss(lpc.astype(np.float64), A, old, objective, el, eh, sc)
    lo, go, ro = loss.cpu().numpy(), g.cpu().numpy(), ratio.cpu().numpy()
    fin = np.isfinite(lpc)
    np.testing.assert_allclose(lo[fin], ref["loss"][fin], rtol=1e-5, atol=1e-7)
    np.testing.assert_allclose(go, ref["g"], rtol=1e-5, atol=1e-7)
    np.testing.assert_allclose(ro, ref["ratio"], rtol=1e-6)
    assert np.isnan(lo[9]) and go[9] == 0.0 and lo[5] == 0.0 and go[5] == 0.0 and ro[5] == 0.0
    # every branch is exercised
    r = ref["ratio"][fin]
    Af = A[fin]
    if objective == "clip":
        clipped = ref["g"][fin] == 0.0
        say(f"  clipped rows {int(clipped.sum())} of {int(fin.sum())}")
        assert clipped.any() and (~clipped).any()
        assert ((Af > 0) & (r > 1 + eh)).any() and ((Af < 0) & (r < 1 - el)).any()
    else:
        assert (r > 1 + eh).any() and (r < 1 + eh).any()


@pytest.mark.parametrize("name,T,V,objective", [("headline", 96, 4096, "cispo"), ("top_p", 128, 6000, "clip"),
                                                ("tiny", 64, None, "clip")])
def test_policy_step_gradients_match_oracle(name, T, V, objective):
    w = workloads.make(name, T=T)
    if V is not None:
        w["W"] = w["W"][:V]
    V = w["W"].shape[0]
    say(f"policy step: {name} T={T} H={w['H']} V={V} {objective}")
    y = targets(w)
    G = to_gpu(w, y)
    keys = binding.scaled_logits(G["h"], G["W"], G["temperature"]).cpu().numpy()   # support on the GPU's keys
    ref = oracle.forward(w["h"], w["W"], y, w["temperature"], w["top_k"], w["top_p"], w["min_p"], keys=keys)
    A, old = _pg_inputs(ref["logprob"], 7)
    el, eh, sc = 0.2, 0.28, 1.0 / T
    loss, lp, ratio, gh, gw = binding.policy_loss_step(
        G["h"], G["W"], G["target"], torch.from_numpy(A).to(dev()), torch.from_numpy(old).to(dev()),
        **meta_of(G), objective=objective, eps_low=el, eps_high=eh, scale=sc)
    pg = oracle.policy_loss(ref["logprob"], A, old, objective, el, eh, sc)
    dH, dW = oracle.backward(w["h"], w["W"], y, ref, pg["g"], w["temperature"])
    rl = abs(float(loss.double().sum()) - pg["loss"].sum()) / max(1e-12, abs(pg["loss"]).sum())
    rh, rw = rel_fro(gh.float().cpu().numpy(), dH), rel_fro(gw.cpu().numpy(), dW)
    say(f"  loss rel {rl:.2e}  dH rel {rh:.2e}  dW rel {rw:.2e}")
    assert rl < 1e-3
    assert rh < GRAD_RTOL and rw < GRAD_RTOL
