"""The autograd wrapper (binding.ScoreFunction) on the GPU, through the C ABI:
its gradients are the library's backward for the incoming gradient, bit for
bit, inside an ordinary torch graph (a weighted sum of logprobs, out-of-support
and inactive rows included), in the default lane, the bf16 lane and with the
scalar pre-GEMM temperature."""
import numpy as np
import pytest
import torch

from gpu_helpers import dev, meta_of, say, targets, to_gpu
from sampling_transform_logprob_amd import binding, workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.load()


@pytest.mark.parametrize("opts", [{}, {"lane": "bf16"}, {"pre_gemm_temperature": 0.6},
                                  {"ignore_index": -100, "lane": "bf16"}])
def test_score_function_gradients_are_the_library_backward(opts):
    T, V = 160, 5000
    w = workloads.make("headline", T=T)
    w["W"] = w["W"][:V]
    y = np.asarray(targets(w), np.int64) % V
    G = to_gpu(w, y)
    if "ignore_index" in opts:
        G["target"][5:9] = opts["ignore_index"]
    meta = meta_of(G)
    if "pre_gemm_temperature" in opts:
        meta["temperature"] = None
    say(f"autograd wrapper: headline T={T} V={V} {opts}")
    h = G["h"].clone().requires_grad_(True)
    W = G["W"].clone().requires_grad_(True)
    lp = binding.ScoreFunction.apply(h, W, G["target"], meta["temperature"], meta["top_k"], meta["top_p"],
                                     meta["min_p"], opts.get("ignore_index"), opts.get("pre_gemm_temperature"),
                                     opts.get("lane", "fp32"))
    adv = torch.linspace(-1.0, 1.0, T, device=dev())
    fin = torch.isfinite(lp)
    loss = -(torch.where(fin, lp, torch.zeros_like(lp)) * adv).sum()
    loss.backward()
    g = torch.where(fin, -adv, torch.zeros_like(adv))
    lp2, st = binding.forward(G["h"], G["W"], G["target"], **meta, **opts)
    gh, gw = binding.backward(G["h"], G["W"], G["target"], st, g, **meta, **opts)
    assert torch.equal(lp.detach().view(torch.int32), lp2.view(torch.int32))
    assert torch.equal(h.grad, gh) and torch.equal(W.grad, gw.to(W.dtype))
    say(f"  bitwise: logprob, grad_hidden, grad_weight; -inf rows {int((~fin).sum())}")
