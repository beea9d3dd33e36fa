"""The backward's recompute product gives the forward's keys bit for bit.

The recompute closed-form VJP re-derives each row's support membership from
keys it recomputes, against the boundary the forward saved, so those keys
must be the forward's exactly.  ``stce_recompute_keys`` launches the
backward's recompute product as ``stce_backward`` does (same kernel, same
vocabulary slices), and that launch also exports the keys it forms.  They
are compared bitwise with the forward projection's keys (``stce_scaled_logits``),
with the target key and the row maximum the forward stored in its per-row
state, over multi-chunk forwards and multi-slice backwards, in every lane
convention."""
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


@pytest.mark.parametrize("name,T,V,chunk,vslice,opts", [
    ("headline", 300, 9000, 64, 2048, {}),                         # 5 chunks, 5 slices (one ragged)
    ("ties", 280, 20000, 100, 6144, {}),                           # tie groups, mixed programs
    ("top_p", 200, 12000, 48, 4096, {"lane": "bf16"}),             # bf16 value lane
    ("headline", 260, 7000, 64, 2560, {"pre_gemm_temperature": 0.7}),
    ("tiny", 64, 1000, 16, 256, {}),                               # fp32 operands
])
def test_recomputed_keys_are_the_forwards(name, T, V, chunk, vslice, opts):
    w = workloads.make(name, T=T)
    w["W"] = w["W"][:V]
    w["V"] = V
    y = targets(w)
    G = to_gpu(w, y)
    meta = meta_of(G)
    if "pre_gemm_temperature" in opts:
        meta["temperature"] = None
    say(f"recompute keys {name}: T={T} V={V} chunk {chunk} slice {vslice} {opts}")
    lp, st = binding.forward(G["h"], G["W"], G["target"], **meta, chunk_rows=chunk, **opts)
    g = torch.from_numpy(np.random.Generator(np.random.PCG64(T)).standard_normal(T).astype(np.float32)).to(dev())
    rk = binding.recompute_keys(G["h"], G["W"], G["target"], st, g, **meta, vocab_slice=vslice, **opts)
    fk = binding.scaled_logits(G["h"], G["W"], meta["temperature"],
                               **{k: v for k, v in opts.items() if k in ("lane", "pre_gemm_temperature")})
    torch.cuda.synchronize()
    prob, _ = binding.make_problem(G["h"], G["W"], G["target"], **meta, vocab_slice=vslice, **opts)
    assert binding.schedule(prob)[1] == vslice < V                 # several vocabulary slices
    assert torch.equal(rk.view(torch.int32), fk.view(torch.int32)), "recomputed keys differ from the forward's"
    info = binding.decode_state(st)
    rkc = rk.cpu()
    sy = rkc[torch.arange(T), G["target"].cpu()].numpy()
    assert np.array_equal(sy.view(np.int32), info["target_key"].view(np.int32))
    assert np.array_equal(rkc.max(1).values.numpy().view(np.int32), info["row_max"].view(np.int32))
    say(f"  {T * V} keys equal; target keys and row maxima equal the forward's state")
