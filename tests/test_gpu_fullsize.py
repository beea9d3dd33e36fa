"""Parity at the full configuration sizes, in the launch configuration the
bench times (default chunk and vocabulary-slice schedule).

The whole forward and backward run on every row.  The oracle then checks
sampled rows one by one:

* the support, bit for bit, decided on the GPU's own keys for those rows;
* logprob and the side outputs;
* the grad_hidden rows, which depend only on their own row.

grad_weight sums over every row, so it is checked through a property that
holds at any size: each row's dz sums to zero over the vocabulary, so the
columns of grad_weight sum to zero.  Rows that are not sampled take the
argmax of their logits (plain torch, fp32), which lies in every support,
except every tenth row, which keeps a uniform target (mostly outside its
support: -inf and zero gradient at scale); the sampled rows get targets
drawn from their filtered distribution.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import GRAD_RTOL, LOGPROB_ATOL, dev, meta_of, rel_fro, say, to_gpu
from sampling_transform_logprob_amd import binding, workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.load()


@pytest.mark.parametrize("name", ["identity", "headline", "top_p", "ties"])
def test_full_size_sampled_rows(name):
    w = workloads.make(name)
    T, H, V = w["T"], w["H"], w["V"]
    rng = np.random.Generator(np.random.PCG64(1234))
    sample = np.unique(np.concatenate([[0, T - 1], rng.choice(T, 8, replace=False)]))
    say(f"full size {name}: T={T} H={H} V={V}, sampled rows {sample.tolist()}")
    y = w["target_uniform"].copy()
    # most rows: the argmax of their logits (plain torch fp32 product; the top token is in every support);
    # every tenth row keeps its uniform target
    G0 = to_gpu(w, y)
    am = torch.cat([(G0["h"][r:r + 2048].float() @ G0["W"].float().T).argmax(1)
                    for r in range(0, T, 2048)]).cpu().numpy()
    del G0
    keep_u = np.arange(T) % 10 == 0
    y = np.where(keep_u, y, am)
    if w["filtered"]:
        y[sample] = oracle.sample_targets(w["h"], w["W"], w["temperature"], w["top_k"], w["top_p"], w["min_p"],
                                          w["u"], rows=sample)
    G = to_gpu(w, y)
    prob, _ = binding.make_problem(G["h"], G["W"], G["target"], **meta_of(G))
    C, Vs = binding.schedule(prob)
    say(f"  schedule: chunk {C} rows, vocabulary slice {Vs}")
    lp, st, side = binding.forward(G["h"], G["W"], G["target"], **meta_of(G), side=True)
    g = torch.full((T,), -1.0 / T, device=dev())
    gh, gw = binding.backward(G["h"], G["W"], G["target"], st, g, **meta_of(G))
    torch.cuda.synchronize()
    # keys of the sampled rows from the same projection kernel (bitwise independent of the row's position)
    si = torch.from_numpy(sample).to(dev())
    keys = binding.scaled_logits(G["h"][si].contiguous(), G["W"], G["temperature"][si].contiguous()).cpu().numpy()
    ref = oracle.forward(w["h"], w["W"], y, w["temperature"], w["top_k"], w["top_p"], w["min_p"], keys=keys,
                         rows=sample)
    info = binding.decode_state(st)
    filt = (info["flags"][sample] & binding.FLAG_FILTERED) != 0
    assert np.array_equal(info["n"][sample], ref["n"])
    assert np.array_equal(info["key_thr"][sample][filt], ref["key_thr"][filt])
    assert np.array_equal(info["id_thr"][sample][filt], ref["id_thr"][filt])
    lpg = lp.cpu().numpy().astype(np.float64)[sample]
    fin = np.isfinite(ref["logprob"])
    assert np.array_equal(np.isfinite(lpg), fin) and fin.all()
    err = np.abs(lpg - ref["logprob"]).max()
    sd = {k: v.cpu().numpy().astype(np.float64)[sample] for k, v in side.items()}
    e_s = max(np.abs(sd["lse_full"] - ref["lse_full"]).max(), np.abs(sd["entropy_support"] - ref["entropy_support"]).max())
    e_f = np.abs(sd["entropy_full"] - ref["entropy_full"]).max()
    dH, _ = oracle.backward(w["h"], w["W"], y, ref, np.full(T, -1.0 / T), w["temperature"])
    rh = rel_fro(gh[si].float().cpu().numpy(), dH)
    colsum = gw.double().sum(0).abs().max().item()
    scale = gw.abs().max().item()
    lpa = lp.cpu().numpy()
    say(f"  logprob err {err:.2e}  side err {e_s:.2e}/{e_f:.2e}  dH rows rel {rh:.2e}  "
        f"|sum_v dW| {colsum:.2e} (max|dW| {scale:.2e})  -inf rows {int(np.isinf(lpa).sum())}")
    assert err < LOGPROB_ATOL and e_s < 1e-4 and e_f < 5e-4 and rh < GRAD_RTOL
    # each term of a column sum is below max|dW|; fp32 dW rounding over V rows bounds the sum
    assert colsum < 1e-3 * scale * np.sqrt(V)
    assert np.isfinite(lpa[~np.isinf(lpa)]).all()
