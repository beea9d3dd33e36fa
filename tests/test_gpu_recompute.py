"""The backward's recompute product gives the forward's keys bit for bit.

The recompute closed-form VJP re-derives each row's support membership from
keys it recomputes, against the boundary the forward saved, so those keys
must be the forward's exactly.  ``stce_recompute_keys`` launches the
backward's recompute product as ``stce_backward`` does (same kernel, same
vocabulary slices, and the tile recompute of the rows with tile lists), and
those launches also export the keys they form.  They are compared bitwise with
the forward projection's keys (``stce_scaled_logits``), with the target key
and the row maximum the forward stored in its per-row state, over
multi-chunk forwards and multi-slice backwards, in every lane convention.
A tiled row's keys are recomputed on its listed tiles only: the list must be
exactly the tiles whose largest key reaches the row's last support key, and
the row's other keys are not formed.  A row whose support the state lists
with its keys has none recomputed: its list must hold the forward's keys of
its support; with the listed flags cleared, the same rows take the tile
recompute, whose keys are checked the same way."""
import numpy as np
import pytest
import torch

from gpu_helpers import (check_recomputed_keys, check_support_lists, check_tile_lists, dev, meta_of, say, targets,
                         to_gpu, unlisted)
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
    st_u = unlisted(st, T)
    rku = binding.recompute_keys(G["h"], G["W"], G["target"], st_u, g, **meta, vocab_slice=vslice, **opts)
    fk = binding.scaled_logits(G["h"], G["W"], meta["temperature"],
                               **{k: v for k, v in opts.items() if k in ("lane", "pre_gemm_temperature")})
    torch.cuda.synchronize()
    prob, _ = binding.make_problem(G["h"], G["W"], G["target"], **meta, vocab_slice=vslice, **opts)
    assert binding.schedule(prob)[1] == vslice < V                 # several vocabulary slices
    info = binding.decode_state(st)
    fkc = fk.cpu().numpy()
    check_tile_lists(info, fkc, V)
    nlisted = check_support_lists(info, fkc)
    nformed, ntiled = check_recomputed_keys(rk.cpu().numpy(), fkc, info, g.cpu().numpy(), y, V, w["dtype"])
    nformed_u, ntiled_u = check_recomputed_keys(rku.cpu().numpy(), fkc, binding.decode_state(st_u),
                                                g.cpu().numpy(), y, V, w["dtype"])
    say(f"  {nlisted} rows list their support with the forward's keys; {nformed} keys equal ({ntiled} tiled "
        f"rows, {T * V - nformed} keys not formed); with the lists unused {nformed_u} keys equal ({ntiled_u} "
        f"tiled rows); target keys and row maxima equal the forward's state")
