"""GPU checks of ignore_index rows (inactive rows, as the cross-entropy VJP of
nested-learning's compute_teach_signal masks them), through the C ABI.

An ignored row scores 0 with an exactly zero gradient and no error; every
other row is bit-identical to the run without the ignored targets; side
outputs of ignored rows are still computed (same bits); the policy loss
reads the state and gives ignored rows zero loss and gradient.  Gradients
against the oracle at the core's bar (1e-2 relative Frobenius)."""
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


@pytest.mark.parametrize("name,T,V", [("top_p", 128, 8000), ("ties", 140, 9000)])
def test_ignored_rows(name, T, V):
    w = workloads.make(name, T=T)
    w["W"] = w["W"][:V]
    say(f"ignore_index: {name} T={T} V={V}")
    y = targets(w)
    yi = y.copy()
    ign = np.zeros(T, bool)
    ign[::7] = True
    yi[ign] = -100
    G = to_gpu(w, y)
    Gi = to_gpu(w, yi)
    lp0, st0, side0 = binding.forward(G["h"], G["W"], G["target"], **meta_of(G), side=True)
    lp, st, side = binding.forward(Gi["h"], Gi["W"], Gi["target"], **meta_of(Gi), side=True, ignore_index=-100)
    lpc, lp0c = lp.cpu(), lp0.cpu()
    assert (lpc[ign] == 0).all()
    assert torch.equal(lpc[~ign].view(torch.int32), lp0c[~ign].view(torch.int32))
    for k in side:
        assert torch.equal(side[k].cpu().view(torch.int32), side0[k].cpu().view(torch.int32)), k
    info = binding.decode_state(st)
    assert ((info["flags"][ign] & binding.FLAG_IGNORED) != 0).all()
    assert ((info["flags"][ign] & binding.FLAG_IN_SUPPORT) == 0).all()
    g = torch.from_numpy(np.random.Generator(np.random.PCG64(3)).standard_normal(T).astype(np.float32)).to(dev())
    gh, gw = binding.backward(Gi["h"], Gi["W"], Gi["target"], st, g, **meta_of(Gi), ignore_index=-100)
    assert not gh[torch.from_numpy(ign).to(dev())].any()
    keys = binding.scaled_logits(G["h"], G["W"], G["temperature"]).cpu().numpy()
    ref = oracle.forward(w["h"], w["W"], yi, w["temperature"], w["top_k"], w["top_p"], w["min_p"], keys=keys,
                         ignore_index=-100)
    dH, dW = oracle.backward(w["h"], w["W"], yi, ref, g.cpu().numpy().astype(np.float64), w["temperature"])
    rh, rw = rel_fro(gh.float().cpu().numpy(), dH), rel_fro(gw.cpu().numpy(), dW)
    say(f"  ignored {int(ign.sum())} rows; dH rel {rh:.2e} dW rel {rw:.2e}")
    assert rh < GRAD_RTOL and rw < GRAD_RTOL
    # the policy loss skips the rows the state marks inactive
    A = torch.ones(T, device=dev())
    old = torch.full((T,), -1.0, device=dev())
    loss, gl, ratio = binding.policy_loss(lp, A, old, "cispo", state=st)
    i = torch.from_numpy(ign).to(dev())
    assert not loss[i].any() and not gl[i].any() and not ratio[i].any()
    assert (gl[~i] != 0).all()
