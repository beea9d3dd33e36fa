"""GPU parity of the forward's side outputs (full-row log-sum-exp, full-row
entropy, filtered-support entropy) against the oracle, through the C ABI.

The oracle decides supports on the GPU's own fp32 keys and computes the
values in fp64 from z / T.  Tolerances follow from the arithmetic:
  * the keys differ from z / T by at most half an fp32 ulp (|s| <= ~40 here,
    so ~2e-6 absolute), which moves an entropy or a log-sum-exp by about as
    much;
  * the full-row quantities come from fp32 per-tile sums of 256 terms
    (relative error up to ~256 * 2^-24 = 1.5e-5 per tile), combined in fp64;
  * the support entropy is summed in fp64 from the keys.
So: lse_full within 1e-4 absolute, entropy_full within 5e-4, entropy_support
within 1e-4.  Asking for the side outputs must not change a single bit of the
logprob or the state.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import meta_of, say, targets, to_gpu
from sampling_transform_logprob_amd import binding, workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.load()


CASES = [("tiny", 64, None), ("identity", 200, None), ("top_p", 200, None), ("headline", 160, 40000),
         ("ties", 200, 30000)]


@pytest.mark.parametrize("name,T,V", CASES)
def test_side_outputs_match_oracle(name, T, V):
    w = workloads.make(name, T=T)
    if V is not None:
        w["W"] = w["W"][:V]
    V = w["W"].shape[0]
    say(f"side outputs {name}: T={T} H={w['H']} V={V}")
    y = targets(w)
    G = to_gpu(w, y)
    lp0, st0 = binding.forward(G["h"], G["W"], G["target"], **meta_of(G))
    lp, st, side = binding.forward(G["h"], G["W"], G["target"], **meta_of(G), side=True)
    assert torch.equal(lp.view(torch.int32), lp0.view(torch.int32)) and torch.equal(st, st0)
    keys = binding.scaled_logits(G["h"], G["W"], G["temperature"]).cpu().numpy()
    ref = oracle.forward(w["h"], w["W"], y, w["temperature"], w["top_k"], w["top_p"], w["min_p"], keys=keys)
    got = {k: v.cpu().numpy().astype(np.float64) for k, v in side.items()}
    e_l = np.abs(got["lse_full"] - ref["lse_full"]).max()
    e_f = np.abs(got["entropy_full"] - ref["entropy_full"]).max()
    e_s = np.abs(got["entropy_support"] - ref["entropy_support"]).max()
    info = binding.decode_state(st)
    say(f"  lse_full err {e_l:.2e}  entropy_full err {e_f:.2e}  entropy_support err {e_s:.2e}  "
        f"support sizes {info['n'].min()}..{info['n'].max()}  H_S range {ref['entropy_support'].min():.3f}.."
        f"{ref['entropy_support'].max():.3f}")
    assert e_l < 1e-4 and e_f < 5e-4 and e_s < 1e-4


def test_side_outputs_of_invalid_rows_are_nan_and_paths_covered():
    w = workloads.make("top_p", T=96)
    w["W"] = w["W"][:20000]
    y = targets(w)
    G = to_gpu(w, y)
    G["top_p"][3] = 0.0                                # invalid row
    G["top_k"][10:20] = 7                              # candidate-window path beside the histogram path
    lp, st, side = binding.forward(G["h"], G["W"], G["target"], **meta_of(G), side=True, check=False)
    for k, v in side.items():
        assert torch.isnan(v[3]), k
    keys = binding.scaled_logits(G["h"], G["W"], G["temperature"]).cpu().numpy()
    ok = np.ones(96, bool)
    ok[3] = False
    tk = G["top_k"].cpu().numpy()
    rows = np.where(ok)[0]
    ref = oracle.forward(w["h"], w["W"], y, w["temperature"], tk, w["top_p"], w["min_p"], keys=keys[rows], rows=rows)
    hs = side["entropy_support"].cpu().numpy().astype(np.float64)[ok]
    assert np.abs(hs - ref["entropy_support"]).max() < 1e-4
    # top-p 0.95 on a 20000-token row keeps thousands of tokens (histogram path, mass ahead of the
    # window: membership pass); top-k 7 rows take the window path
    n = ref["n"]
    assert n.max() > 1000 and (n[(rows >= 10) & (rows < 20)] == 7).all()
