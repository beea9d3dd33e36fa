"""stce_forward_noalloc, the forward that allocates nothing (its workspace
is the library's static device array), against stce_forward: logprob and
state bit for bit, on two calls in a row on the shared array, the second
smaller, and on a problem that takes several chunks to fit the array."""
import numpy as np
import pytest
import torch

from gpu_helpers import meta_of, say, targets, to_gpu
from sampling_transform_logprob_amd import binding, workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.load()


def _pair(name, T, V, **kw):
    w = workloads.make(name, T=T)
    if V is not None:
        w["W"] = w["W"][:V]
        w["V"] = V
    y = targets(w)
    G = to_gpu(w, y)
    lp, st = binding.forward(G["h"], G["W"], G["target"], **meta_of(G), **kw)
    lpn, stn = binding.forward_noalloc(G["h"], G["W"], G["target"], **meta_of(G), **kw)
    torch.cuda.synchronize()
    return lp, st, lpn, stn


def test_noalloc_forward_equals_forward_on_two_calls():
    assert binding.load().stce_noalloc_scratch_bytes() == 64 << 20
    # first call: 600 rows of the headline program over 40,000 tokens (the
    # workspace of one 600-row chunk exceeds the array: several chunks)
    lp, st, lpn, stn = _pair("headline", 600, 40000)
    assert torch.equal(lp.view(torch.int32), lpn.view(torch.int32)) and torch.equal(st, stn)
    # second call, smaller, on the array the first call left behind
    lp, st, lpn, stn = _pair("ties", 96, 9000)
    assert torch.equal(lp.view(torch.int32), lpn.view(torch.int32)) and torch.equal(st, stn)
    # fp32 operands, every filter mixed, a chunk size of the caller's
    lp, st, lpn, stn = _pair("tiny", 64, None, chunk_rows=16)
    assert torch.equal(lp.view(torch.int32), lpn.view(torch.int32)) and torch.equal(st, stn)
    say("noalloc forward: bitwise equal to stce_forward on three calls")
