"""The backward's row classes: rows whose support holds at most NSP = 128
tokens take the sparse products (their dz entries summed one by one), larger
supports the matrix-core products, rows with no gradient neither.  A sparse
row's entries come from the support the state lists with its keys, else
from its keys recomputed on its listed tiles, else from the whole-vocabulary
recompute; the three give the same entries.  Every mix is held to the oracle
(gradients within 1e-2 relative Frobenius error) and to run-to-run bitwise
equality."""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import (GRAD_RTOL, check_support_lists, check_tile_lists, dev, listed_rows, meta_of, rel_fro, say,
                         targets, tiled_rows, to_gpu, unlisted, without_lists)
from sampling_transform_logprob_amd import binding, workloads
from sampling_transform_logprob_amd.workloads import round_bf16

pytestmark = pytest.mark.gpu

NSP = 128


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.load()


def _oracle_grads(w, y, g, keys):
    ref = oracle.forward(w["h"], w["W"], y, w["temperature"], w["top_k"], w["top_p"], w["min_p"], keys=keys)
    return ref, oracle.backward(w["h"], w["W"], y, ref, g, w["temperature"])


def test_mixed_classes_and_the_class_boundary():
    """One batch with every class: top-k NSP and NSP + 1 (the two sides of
    the class boundary), top-p over most of the row (dense), top-k 20
    (sparse), unfiltered rows (dense), targets out of support and a zero
    upstream gradient (empty); several vocabulary slices."""
    T, V = 240, 12000
    w = workloads.make("headline", T=T)
    w["W"] = w["W"][:V]
    w["V"] = V
    kind = np.arange(T) % 6
    w["top_k"] = np.select([kind == 0, kind == 1, kind == 2, kind == 3], [NSP, NSP + 1, 20, 0], 0).astype(np.int32)
    w["top_p"] = np.where(kind == 4, 0.95, 1.0).astype(np.float32)
    w["min_p"] = np.zeros(T, np.float32)
    y = targets(w)
    y[kind == 5] = w["target_uniform"][kind == 5] % V                 # unfiltered rows
    G0 = to_gpu(w, y)
    keys = binding.scaled_logits(G0["h"], G0["W"], G0["temperature"]).cpu().numpy()
    out = np.nonzero(kind == 2)[0][::3]                                # some top-20 rows: target out of support
    for r in out:
        y[r] = int(oracle.order_row(keys[r])[-1])
    g = np.random.Generator(np.random.PCG64(5)).standard_normal(T)
    g[7::17] = 0.0                                                     # zero upstream gradient
    G = to_gpu(w, y)
    say(f"classes: T={T} V={V}")
    lp, st = binding.forward(G["h"], G["W"], G["target"], **meta_of(G))
    gg = torch.from_numpy(g.astype(np.float32)).to(dev())
    gh, gw = binding.backward(G["h"], G["W"], G["target"], st, gg, **meta_of(G), vocab_slice=4096)
    gh2, gw2 = binding.backward(G["h"], G["W"], G["target"], st, gg, **meta_of(G), vocab_slice=4096)
    torch.cuda.synchronize()
    assert torch.equal(gh, gh2) and torch.equal(gw, gw2)
    info = binding.decode_state(st)
    n = info["n"]
    assert (n[kind == 0] == NSP).all() and (n[kind == 1] == NSP + 1).all()
    ref, (dH, dW) = _oracle_grads(w, y, g, keys)
    assert np.array_equal(n, ref["n"])
    rh, rw = rel_fro(gh.float().cpu().numpy(), dH), rel_fro(gw.cpu().numpy(), dW)
    say(f"  dH rel {rh:.2e} dW rel {rw:.2e}; out-of-support rows {int((~ref['in_support']).sum())}")
    assert rh < GRAD_RTOL and rw < GRAD_RTOL
    ghc = gh.float().cpu().numpy()
    assert not ghc[~ref["in_support"]].any() and not ghc[g == 0].any()


def test_accumulate_and_single_outputs():
    """Sparse rows only (top-k 20): the weight gradient added onto the
    caller's array, and each gradient requested alone."""
    T, V = 200, 9000
    w = workloads.make("headline", T=T)
    w["W"] = w["W"][:V]
    w["V"] = V
    y = targets(w)
    G = to_gpu(w, y)
    lp, st = binding.forward(G["h"], G["W"], G["target"], **meta_of(G))
    g = torch.full((T,), -1.0 / T, device=dev())
    gh, gw = binding.backward(G["h"], G["W"], G["target"], st, g, **meta_of(G))
    base = torch.randn(V, w["H"], device=dev())
    _, acc = binding.backward(G["h"], G["W"], G["target"], st, g, **meta_of(G), need_hidden=False,
                              grad_weight=base.clone(), accumulate_grad_weight=True)
    gh_only, none_w = binding.backward(G["h"], G["W"], G["target"], st, g, **meta_of(G), need_weight=False)
    none_h, gw_only = binding.backward(G["h"], G["W"], G["target"], st, g, **meta_of(G), need_hidden=False)
    torch.cuda.synchronize()
    assert none_w is None and none_h is None
    assert torch.equal(gh_only, gh) and torch.equal(gw_only, gw)
    assert torch.allclose(acc, base + gw, rtol=0, atol=1e-6)
    rows_hit = (gw != 0).any(1)
    assert torch.equal(acc[~rows_hit], base[~rows_hit])            # untouched rows keep the caller's values
    say(f"  accumulate: {int(rows_hit.sum())} vocabulary rows receive sparse terms")


def test_a_token_in_every_support_takes_the_windowed_bucket():
    """One vocabulary row dominates every logit row, so it lies in all 5000
    supports: its weight-gradient bucket (5000 entries) exceeds the 1024 the
    kernel orders in LDS and is summed window by window of positions."""
    rng = np.random.Generator(np.random.PCG64(8))
    T, H, V = 5000, 64, 3000
    h = round_bf16(rng.standard_normal((T, H)).astype(np.float32) + 2.0)
    W = round_bf16((rng.standard_normal((V, H)) * 0.05).astype(np.float32))
    W[17] = round_bf16(np.full(H, 0.05, np.float32))                 # h . W[17] ~ 6.4: in every top-8
    w = dict(h=h, W=W, temperature=np.full(T, 0.9, np.float32), top_k=np.full(T, 8, np.int32),
             top_p=np.ones(T, np.float32), min_p=np.zeros(T, np.float32), dtype="bf16", u=rng.random(T),
             filtered=True, V=V)
    y = targets(w)
    g = rng.standard_normal(T)
    G = to_gpu(w, y)
    lp, st = binding.forward(G["h"], G["W"], G["target"], **meta_of(G))
    gg = torch.from_numpy(g.astype(np.float32)).to(dev())
    gh, gw = binding.backward(G["h"], G["W"], G["target"], st, gg, **meta_of(G))
    gh2, gw2 = binding.backward(G["h"], G["W"], G["target"], st, gg, **meta_of(G))
    keys = binding.scaled_logits(G["h"], G["W"], G["temperature"]).cpu().numpy()
    torch.cuda.synchronize()
    assert torch.equal(gw, gw2) and torch.equal(gh, gh2)
    assert (keys.argmax(1) == 17).all()                              # so token 17 is in every support
    ref, (dH, dW) = _oracle_grads(w, y, g, keys)
    rh, rw = rel_fro(gh.float().cpu().numpy(), dH), rel_fro(gw.cpu().numpy(), dW)
    say(f"windowed bucket: T={T} dH rel {rh:.2e} dW rel {rw:.2e} (row 17 rel "
        f"{rel_fro(gw[17].cpu().numpy(), dW[17]):.2e})")
    assert rh < GRAD_RTOL and rw < GRAD_RTOL
    assert rel_fro(gw[17].cpu().numpy(), dW[17]) < GRAD_RTOL     # the windowed row itself (dz is bf16)


@pytest.mark.parametrize("name,T,V", [("headline", 300, 30000), ("headline_fp8", 260, 20000), ("ties", 280, 20000)])
def test_listed_tiled_and_whole_vocabulary_entries_agree(name, T, V):
    """A sparse row whose support the state lists takes its dz entries from
    the listed keys; the same state with the listed flags cleared recomputes
    its keys on its listed tiles, and with the tile lists cleared too in the
    whole-vocabulary recompute.  All three must give the same entries.  dH
    sums a row's entries in vocabulary order, so it is bitwise equal; dW
    sums a vocabulary row's entries in permuted-position order, which the
    three placements keep when every sparse row is listed and tiled (then
    dW is bitwise equal) and otherwise change (equal up to fp32 summation
    order)."""
    w = workloads.make(name, T=T)
    w["W"] = w["W"][:V]
    if w.get("w_scale") is not None:
        w["w_scale"] = w["w_scale"][:V]
    w["V"] = V
    y = targets(w)
    G = to_gpu(w, y)
    ws = {"weight_scale": G["weight_scale"]} if G["weight_scale"] is not None else {}
    lp, st = binding.forward(G["h"], G["W"], G["target"], **meta_of(G), **ws)
    g = torch.from_numpy(np.random.Generator(np.random.PCG64(T)).standard_normal(T).astype(np.float32)).to(dev())
    st_tiled, st_full = unlisted(st, T), without_lists(st, T)
    gh, gw = binding.backward(G["h"], G["W"], G["target"], st, g, **meta_of(G), **ws, vocab_slice=8192)
    gh1, gw1 = binding.backward(G["h"], G["W"], G["target"], st_tiled, g, **meta_of(G), **ws, vocab_slice=8192)
    gh0, gw0 = binding.backward(G["h"], G["W"], G["target"], st_full, g, **meta_of(G), **ws, vocab_slice=8192)
    # the problem flag that ignores the lists: the listed flags cleared
    ghr, gwr = binding.backward(G["h"], G["W"], G["target"], st, g, **meta_of(G), **ws, vocab_slice=8192,
                                recompute_all=True)
    keys = binding.scaled_logits(G["h"], G["W"], G["temperature"], **ws).cpu().numpy()
    torch.cuda.synchronize()
    info = binding.decode_state(st)
    gc = g.cpu().numpy()
    nlisted = check_support_lists(info, keys)
    listed = listed_rows(info, gc, w["dtype"])
    tiled = tiled_rows(binding.decode_state(st_tiled), gc, V, w["dtype"])
    say(f"listed / tiled / whole-vocabulary {name}: T={T} V={V}: {nlisted} rows list their support "
        f"({int(listed.sum())} with a gradient); without the lists {int(tiled.sum())} tiled rows, "
        f"{int(info['ntile'][tiled].sum())} (row, tile) pairs of {T * (-(-V // 256))}")
    assert listed.sum() > (T // 3 if name != "ties" else 0) and tiled.sum() > (T // 3 if name != "ties" else 0)
    assert torch.equal(gh, gh1) and torch.equal(gh, gh0)
    assert torch.equal(ghr, gh1) and torch.equal(gwr, gw1)
    fl = info["flags"]
    active = ((fl & binding.FLAG_VALID) != 0) & ((fl & binding.FLAG_IN_SUPPORT) != 0) & (gc != 0)
    sparse = active & ((fl & binding.FLAG_FILTERED) != 0) & (info["n"] <= NSP)
    for other, label in ((gw1, "tiled"), (gw0, "whole-vocabulary")):
        if np.array_equal(sparse, listed) and np.array_equal(sparse, tiled):
            assert torch.equal(gw, other), label
        else:
            err = (gw - other).abs().max().item() / other.abs().max().item()
            say(f"  dW against the {label} path: placement differs; max difference {err:.1e} of the largest entry")
            assert err < 1e-5, label


def test_tile_lists_at_the_31_tile_bound():
    """Rows whose support spans 30, 31 and 32 vocabulary tiles: one peak
    token per tile (distinct heights, far above the rest), top-k equal to
    the number of peaks.  The lists hold 30 and 31 tiles; a 32-tile support
    keeps no list.  The rows list their supports; with the listed flags
    cleared the 30- and 31-tile rows take the tile recompute and the 32-tile
    rows the whole-vocabulary one.  Every path agrees with the oracle and
    with the lists cleared."""
    rng = np.random.Generator(np.random.PCG64(31))
    ntv, H = 40, 64
    V = ntv * 256
    T = H                                                  # one hidden coordinate per row
    m_of = np.array([30, 31, 32])[np.arange(T) % 3]
    # row r's hidden state is the unit vector e_r, so its keys are column r
    # of W: small noise, and one peak per chosen tile, of distinct heights
    h = np.eye(T, H, dtype=np.float32)
    W = (rng.standard_normal((V, H)) * 0.01).astype(np.float32)
    for r in range(T):
        tiles = rng.choice(ntv, m_of[r], replace=False)
        toks = tiles * 256 + rng.integers(0, 256, m_of[r])
        W[toks, r] = 5.0 + 0.25 * np.arange(m_of[r], dtype=np.float32)   # bf16-exact heights
    h, W = round_bf16(h), round_bf16(W)
    w = dict(h=h, W=W, temperature=np.ones(T, np.float32), top_k=m_of.astype(np.int32),
             top_p=np.ones(T, np.float32), min_p=np.zeros(T, np.float32), dtype="bf16",
             u=rng.random(T), filtered=True, V=V)
    y = targets(w)
    G = to_gpu(w, y)
    lp, st = binding.forward(G["h"], G["W"], G["target"], **meta_of(G))
    g = torch.from_numpy(rng.standard_normal(T).astype(np.float32)).to(dev())
    gh, gw = binding.backward(G["h"], G["W"], G["target"], st, g, **meta_of(G))
    gh1, gw1 = binding.backward(G["h"], G["W"], G["target"], unlisted(st, T), g, **meta_of(G))
    gh0, gw0 = binding.backward(G["h"], G["W"], G["target"], without_lists(st, T), g, **meta_of(G))
    keys = binding.scaled_logits(G["h"], G["W"], G["temperature"]).cpu().numpy()
    torch.cuda.synchronize()
    info = binding.decode_state(st)
    check_tile_lists(info, keys, V)
    check_support_lists(info, keys)
    assert np.array_equal(info["n"], m_of)
    assert np.array_equal(info["ntile"], np.where(m_of <= 31, m_of, 0))
    ref, (dH, dW) = _oracle_grads(w, y, g.cpu().numpy(), keys)
    rh, rw = rel_fro(gh.float().cpu().numpy(), dH), rel_fro(gw.cpu().numpy(), dW)
    say(f"31-tile bound: lists {sorted(set(info['ntile'].tolist()))}; dH rel {rh:.2e} dW rel {rw:.2e}")
    assert rh < GRAD_RTOL and rw < GRAD_RTOL
    rh1, rw1 = rel_fro(gh1.float().cpu().numpy(), dH), rel_fro(gw1.cpu().numpy(), dW)
    assert rh1 < GRAD_RTOL and rw1 < GRAD_RTOL                       # the tile recompute (lists unused)
    assert torch.equal(gh, gh0) and torch.equal(gh, gh1)
    assert (gw - gw0).abs().max().item() <= 1e-5 * gw0.abs().max().item()
    assert (gw - gw1).abs().max().item() <= 1e-5 * gw1.abs().max().item()
