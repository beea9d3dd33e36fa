"""Top-k-bounded rows keep per-tile candidates instead of their fp32 keys.

The projection keeps, per (row, 256-token tile), the two largest keys of each
of the 8 lanes that hold the tile's logits and the largest key that is not a
candidate; the selection decides such a row from the candidates when every
candidate tile's bound lies below the k-th largest tile maximum (and, with
top-p on, when the crossing is the same for every row mass within the
partials' error), else the row is projected again with its keys stored and
selected from them.  Both routes must give the oracle's support bit for bit
on the GPU's own keys."""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import check_logprob, check_support, dev, meta_of, rel_fro, say, targets, to_gpu
from sampling_transform_logprob_amd import binding, workloads
from sampling_transform_logprob_amd.workloads import round_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.load()


def _crowded(T, H, V, seed):
    """Half the rows put their 4 largest logits on tokens 0..3, which one
    lane of tile 0 holds (rows 0..3 of the tile's first 16-row block), so
    that lane's third key reaches the top-20 bound: those rows need the
    re-projection; the other half are ordinary rows."""
    rng = np.random.Generator(np.random.PCG64(seed))
    W = (rng.standard_normal((V, H)) * 0.02).astype(np.float32)
    u = rng.standard_normal(H).astype(np.float32)
    u /= np.linalg.norm(u)
    W[:4] = u[None, :] * np.float32([0.9, 0.85, 0.8, 0.75])[:, None]
    h = rng.standard_normal((T, H)).astype(np.float32)
    crowd = np.arange(T) % 2 == 0
    h[crowd] += (8.0 * u)[None, :]                      # h . W[0..3] ~ 6-7: far above the rest
    return round_bf16(h), round_bf16(W), crowd


@pytest.mark.parametrize("opts", [{}, {"side": True}, {"lane": "bf16"}, {"pre_gemm_temperature": 0.7}])
def test_rows_the_candidates_cannot_decide_are_reprojected(opts):
    T, H, V = 300, 256, 40000
    h, W, crowd = _crowded(T, H, V, 3)
    temp = np.full(T, 0.7, np.float32)
    w = dict(h=h, W=W, temperature=temp, top_k=np.full(T, 20, np.int32), top_p=np.full(T, 0.9, np.float32),
             min_p=np.zeros(T, np.float32), dtype="bf16", u=np.random.Generator(np.random.PCG64(4)).random(T),
             filtered=True, V=V)
    pre = opts.get("pre_gemm_temperature")
    lane = opts.get("lane", "fp32")
    if pre is not None:
        w["temperature"] = np.ones(T, np.float32)
    y = targets(w) if pre is None and lane == "fp32" else np.zeros(T, np.int64)
    G = to_gpu(w, y)
    meta = meta_of(G)
    kw = {k: v for k, v in opts.items() if k in ("lane", "pre_gemm_temperature")}
    if pre is not None:
        meta["temperature"] = None
    say(f"candidates with re-projection: T={T} V={V} {opts}")
    out = binding.forward(G["h"], G["W"], G["target"], **meta, chunk_rows=128, side=opts.get("side", False), **kw)
    lp, st = out[0], out[1]
    keys = binding.scaled_logits(G["h"], G["W"], meta["temperature"], **kw)
    torch.cuda.synchronize()
    kc = keys.cpu().numpy()
    hh = oracle.pre_gemm_hidden(h, pre) if pre is not None else h
    ref = oracle.forward(hh, W, y, w["temperature"], w["top_k"], w["top_p"], w["min_p"], keys=kc, lane=lane)
    info = binding.decode_state(st)
    assert check_support(info, ref, "crowded") == 0
    check_logprob(lp.cpu().numpy(), ref)
    assert (kc[crowd].argsort(1)[:, -4:] < 4).all()      # the crowded rows' top 4 are tokens 0..3
    if opts.get("side"):
        sd = out[2]
        assert np.abs(sd["lse_full"].cpu().numpy() - ref["lse_full"]).max() < 1e-4
        assert np.abs(sd["entropy_support"].cpu().numpy() - ref["entropy_support"]).max() < 1e-4
    # bitwise the same as a forward whose chunks hold one row each (every chunk re-projects or not alone)
    lp1, st1 = binding.forward(G["h"][:40], G["W"], G["target"][:40],
                               **{k: (v[:40] if v is not None else None) for k, v in meta.items()}, chunk_rows=1,
                               **kw)
    assert torch.equal(lp1.view(torch.int32), lp[:40].view(torch.int32)) and torch.equal(st1, binding.state_prefix(st, 40))


def test_top_p_near_the_crossing_is_reselected_from_keys():
    """Rows whose top-p crossing lies within the partials' error of the
    row mass cannot be decided from candidates and are re-projected; rows
    clear of it are decided from the candidates.  fp32 operands with one-hot
    hidden rows make every key an exact column of W."""
    rng = np.random.Generator(np.random.PCG64(17))
    V, H = 20000, 8
    cols = rng.standard_normal((V, H)).astype(np.float32)
    top = rng.choice(V, (H, 2), replace=False)
    for c in range(H):
        cols[top[c], c] = 10.0
    s64 = cols.T.astype(np.float64)
    frac = np.exp(s64[np.arange(H)[:, None], top] - 10.0).sum(1) / np.exp(s64 - 10.0).sum(1)
    rel = np.array([-3e-4, -1e-5, -1e-7, 1e-7, 1e-5, 3e-4, -5e-3, 5e-3])
    T = 64
    c_of = np.arange(T) % H
    p = (frac[c_of] * (1 + rel[(np.arange(T) // H) % 8])).astype(np.float32)
    h = np.zeros((T, H), np.float32)
    h[np.arange(T), c_of] = 1.0
    w = dict(h=h, W=cols, temperature=np.ones(T, np.float32), top_k=np.full(T, 2, np.int32), top_p=p,
             min_p=np.zeros(T, np.float32), dtype="f32", filtered=True, V=V)
    y = top[c_of, 0]
    G = to_gpu(w, y)
    lp, st = binding.forward(G["h"], G["W"], G["target"], **meta_of(G))
    keys = binding.scaled_logits(G["h"], G["W"], G["temperature"]).cpu().numpy()
    ref = oracle.forward(h, cols, y, w["temperature"], w["top_k"], w["top_p"], w["min_p"], keys=keys)
    info = binding.decode_state(st)
    assert check_support(info, ref, "top-p band") == 0
    check_logprob(lp.cpu().numpy(), ref)
    say(f"top-p band through the candidates: supports {sorted(set(info['n'].tolist()))}")


@pytest.mark.parametrize("name,T", [("headline", 256), ("headline_sharp", 256), ("ties", 256)])
def test_candidate_forward_is_the_keys_forward(name, T):
    """The same rows scored with candidates (top-k on) and, row for row,
    with their keys stored: the selection kernel run on the stored keys
    (stce_support_from_logits) gives the same support, flags, row maximum and
    target key, and, on filtered rows (whose log-sum-exp the selection sums
    from the keys), the same filtered log-sum-exp and logprob bits.  (An
    unfiltered row's log-sum-exp comes from the tile partials, which the two
    entries form with different exp arithmetic.)"""
    w = workloads.make(name, T=T)
    assert w["V"] % 4 == 0
    y = targets(w)
    G = to_gpu(w, y)
    lp, st = binding.forward(G["h"], G["W"], G["target"], **meta_of(G))
    keys = binding.scaled_logits(G["h"], G["W"], G["temperature"])
    lp2, st2 = binding.support_from_logits(keys, G["target"], G["top_k"], G["top_p"], G["min_p"])
    torch.cuda.synchronize()
    i1, i2 = binding.decode_state(st), binding.decode_state(st2)
    for f in ("key_thr", "id_thr", "n", "flags", "row_max", "target_key"):
        assert np.array_equal(i1[f].view(np.uint32), i2[f].view(np.uint32)), (name, f)
    filt = (i1["flags"] & binding.FLAG_FILTERED) != 0
    assert np.array_equal(i1["lse_support"][filt].view(np.uint32), i2["lse_support"][filt].view(np.uint32))
    assert np.array_equal(lp.cpu().numpy()[filt].view(np.uint32), lp2.cpu().numpy()[filt].view(np.uint32))
    say(f"candidates vs keys {name}: state and logprob bitwise equal on {int(filt.sum())} filtered rows of {T}")
