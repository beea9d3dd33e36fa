"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: exact
rational arithmetic, brute force on tiny rows, closed forms, a textbook
library routine (log_softmax, autograd), central finite differences and
invariants.  The rules come from xorl pull request 74 ("What this PR does"
item 1: temperature first, stable token-id tie-break, inclusive top-p
crossing, min-p against the original row maximum, top_p == 1 as the exact
identity; item 4: out-of-support targets score -inf with zero gradient;
self-review pass: logprob clamped to <= 0, per-row post-projection
temperature) and from align "architecture v2: proposal" 5.4 A (gradient
``softmax - onehot`` and its sign).
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


# ---------------------------------------------------------------- keys
def test_order_keys_preserve_float_order(rng):
    vals = np.concatenate([
        rng.standard_normal(2000).astype(np.float32) * 50,
        np.array([0.0, -0.0, 1e-45, -1e-45, 3.4e38, -3.4e38, 1.0, -1.0], np.float32),
    ])
    keys = oracle.order_keys(vals).astype(np.int64)
    for _ in range(5000):
        i, j = rng.integers(0, len(vals), 2)
        a, b = float(vals[i]), float(vals[j])
        assert (a < b) == (keys[i] < keys[j]) and (a == b) == (keys[i] == keys[j])
    assert oracle.order_keys(np.array([-0.0], np.float32))[0] == oracle.order_keys(np.array([0.0], np.float32))[0]


def _f32_round_exact(q: Fraction) -> np.float32:
    """Correct rounding of an exact rational to fp32, ties to even (brute)."""
    c = np.float32(float(q))
    best = None
    for cand in (np.nextafter(c, np.float32(-np.inf)), c, np.nextafter(c, np.float32(np.inf))):
        err = abs(Fraction(float(cand)) - q)
        even = (cand.view(np.uint32) & 1) == 0
        if best is None or err < best[0] or (err == best[0] and even):
            best = (err, cand)
    return best[1]


def test_temperature_division_is_correctly_rounded(rng):
    z = (rng.standard_normal(3000) * 10).astype(np.float32)
    t = rng.uniform(0.05, 3.0, 3000).astype(np.float32)
    s = oracle.scale_logits(z[:, None].astype(np.float64), t)[:, 0]
    for i in range(len(z)):
        want = _f32_round_exact(Fraction(float(z[i])) / Fraction(float(t[i])))
        if want == 0:
            want = np.float32(0.0)
        assert s[i].view(np.uint32) == want.view(np.uint32), (z[i], t[i])


def test_temperature_one_is_exact(rng):
    z = (rng.standard_normal((3, 50)) * 7).astype(np.float32).astype(np.float64)
    s = oracle.scale_logits(z, np.ones(3, np.float32))
    assert np.array_equal(s, oracle.canonical_f32(z.astype(np.float32)))


def test_projection_is_exact_on_small_integers(rng):
    h = rng.integers(-9, 10, (3, 7)).astype(np.float32)
    W = rng.integers(-9, 10, (5, 7)).astype(np.float32)
    z = oracle.chunk_logits(h, W)
    for t in range(3):
        for j in range(5):
            assert z[t, j] == sum(int(h[t, c]) * int(W[j, c]) for c in range(7))


# ---------------------------------------------------------------- order and support, brute force
def _precedes(s, i, j):
    return s[i] > s[j] or (s[i] == s[j] and i < j)


def _brute_order(s):
    V = len(s)
    rank = [sum(_precedes(s, j, i) for j in range(V)) for i in range(V)]
    out = [0] * V
    for i, r in enumerate(rank):
        out[r] = i
    return out


def _brute_support(s32, k, p, mp):
    """Support by definition, written without sorting or running sums."""
    s = [float(x) for x in oracle.canonical_f32(s32)]
    V = len(s)
    order = _brute_order(s)
    m = max(s)
    w = [math.exp(x - m) for x in s]
    Z = math.fsum(w)
    sizes = [V]
    if 0 < k < V:
        sizes.append(k)
    if p < 1:
        for n in range(1, V + 1):                       # shortest prefix reaching p of the mass
            if math.fsum(w[order[r]] for r in range(n)) >= float(np.float32(p)) * Z:
                sizes.append(n)
                break
    if mp > 0:
        keep = [i for i in range(V) if s[i] - m >= math.log(float(np.float32(mp)))]
        assert set(keep) == set(order[:len(keep)])      # min-p keeps a prefix
        sizes.append(len(keep))
    n = min(sizes)
    return n, order[n - 1]


def test_order_matches_pairwise_definition(rng):
    for _ in range(200):
        V = int(rng.integers(1, 12))
        s = rng.integers(-3, 4, V).astype(np.float32) * np.float32(0.5)   # many ties
        assert list(oracle.order_row(s)) == _brute_order([float(x) for x in s])


def test_support_matches_brute_force(rng):
    checked = 0
    for _ in range(600):
        V = int(rng.integers(1, 11))
        s = (rng.standard_normal(V) * 2).astype(np.float32)
        if rng.random() < 0.3:
            s = np.round(s).astype(np.float32)                      # ties
        k = int(rng.choice([0, 1, 2, 3, V, V + 3]))
        p = float(rng.choice([1.0, 0.3, 0.6, 0.9, 0.99]))
        mp = float(rng.choice([0.0, 0.05, 0.3, 0.9, 1.0]))
        d = oracle.support_row(s, k, p, mp)
        if d["near"]:
            continue
        n, b = _brute_support(s, k, p, mp)
        assert (d["n"], d["id_thr"]) == (n, b), (s, k, p, mp)
        checked += 1
    assert checked > 500


# ---------------------------------------------------------------- rules, closed forms
def test_top_k_one_is_lowest_argmax_and_logprob_zero():
    s = np.array([1.0, 3.0, 3.0, -2.0], np.float32)
    d = oracle.support_row(s, 1, 1.0, 0.0)
    assert d["n"] == 1 and d["id_thr"] == int(np.argmax(s)) == 1
    h = np.ones((1, 4), np.float32)                   # z = h W^T = s
    W = np.diag(s).astype(np.float32)
    f = oracle.forward(h, W, np.array([1]), top_k=np.array([1]))
    assert f["logprob"][0] == 0.0 and f["n"][0] == 1


def test_top_k_at_least_vocab_is_identity(rng):
    s = (rng.standard_normal(37) * 3).astype(np.float32)
    ref = oracle.support_row(s, 0, 1.0, 0.0)
    for k in (37, 38, 1000):
        d = oracle.support_row(s, k, 1.0, 0.0)
        assert (d["n"], d["id_thr"]) == (ref["n"], ref["id_thr"]) == (37, ref["pi"][-1])


def test_tie_group_split_by_token_id():
    # keys: 5 at ids 0 and 4; 2 at ids 1, 2, 6; 0 at 3 and 5
    s = np.array([5, 2, 2, 0, 5, 0, 2], np.float32)
    d = oracle.support_row(s, 3, 1.0, 0.0)           # {0, 4} then the lowest id of the 2-group
    assert d["n"] == 3 and d["id_thr"] == 1
    mask = oracle.in_support(s, d["key_thr"], d["id_thr"])
    assert set(np.nonzero(mask)[0]) == {0, 4, 1}


def test_top_p_includes_crossing_token():
    prob = np.array([0.5, 0.3, 0.2])
    s = np.log(prob).astype(np.float32)
    # masses before each token: 0, 0.5, 0.8 (up to rounding of the keys)
    assert oracle.support_row(s, 0, 0.45, 0.0)["n"] == 1
    assert oracle.support_row(s, 0, 0.55, 0.0)["n"] == 2     # token 1 crosses 0.55: kept
    assert oracle.support_row(s, 0, 0.79, 0.0)["n"] == 2
    assert oracle.support_row(s, 0, 0.85, 0.0)["n"] == 3


def _overshoot_row():
    """A row whose fp32 running sum of fp32 softmax probabilities (in order)
    reaches 1.0 before its last token: a running-sum test with p = 1 would
    drop the tail."""
    g = np.random.Generator(np.random.PCG64(7))
    while True:
        V = int(g.integers(3, 300))
        s = (g.standard_normal(V) * g.uniform(0.1, 3)).astype(np.float32)
        e = np.exp(s - s.max()).astype(np.float32)
        q = np.sort(e / e.sum(dtype=np.float32))[::-1].astype(np.float32)
        c = np.cumsum(q, dtype=np.float32)
        hit = np.nonzero(c >= np.float32(1.0))[0]
        if hit.size and hit[0] < V - 2:
            return s


def test_top_p_one_is_full_support_despite_fp32_overshoot():
    s = _overshoot_row()
    V = len(s)
    d = oracle.support_row(s, 0, 1.0, 0.0)
    assert d["n"] == V and d["id_thr"] == int(oracle.order_row(s)[-1])


def test_min_p_closed_form_matches_probability_space(rng):
    from scipy.special import softmax
    for _ in range(200):
        V = int(rng.integers(2, 300))
        s = (rng.standard_normal(V) * 2).astype(np.float32)
        mp = float(np.float32(rng.choice([0.01, 0.1, 0.5, 0.9])))
        d = oracle.support_row(s, 0, 1.0, mp)
        if d["near"]:
            continue
        prob = softmax(s.astype(np.float64))
        assert d["n"] == int(np.count_nonzero(prob >= mp * prob.max() * (1 - 1e-13)))


def test_min_p_one_keeps_the_whole_max_tie_group():
    s = np.array([1.0, 4.0, 2.0, 4.0, 4.0], np.float32)
    d = oracle.support_row(s, 0, 1.0, 1.0)
    assert d["n"] == 3 and d["id_thr"] == 4


def test_min_p_never_splits_a_tie_group(rng):
    for _ in range(100):
        V = 40
        s = rng.integers(-4, 4, V).astype(np.float32)
        d = oracle.support_row(s, 0, 1.0, float(np.float32(np.exp(-rng.uniform(0, 6)))))
        kept = oracle.in_support(s, d["key_thr"], d["id_thr"])
        for val in np.unique(s):
            grp = kept[s == val]
            assert grp.all() or not grp.any()


def test_filters_compose_as_shortest_prefix(rng):
    for _ in range(300):
        V = int(rng.integers(2, 60))
        s = (rng.standard_normal(V) * 2).astype(np.float32)
        k, p, mp = int(rng.integers(0, V + 2)), float(rng.uniform(0.05, 1.0)), float(rng.uniform(0, 0.5))
        d = oracle.support_row(s, k, p, mp)
        parts = [oracle.support_row(s, k, 1.0, 0.0)["n"], oracle.support_row(s, 0, p, 0.0)["n"],
                 oracle.support_row(s, 0, 1.0, mp)["n"]]
        assert d["n"] == min(parts)


def test_support_invariants(rng):
    for _ in range(200):
        V = int(rng.integers(1, 200))
        s = (rng.standard_normal(V) * rng.uniform(0.1, 5)).astype(np.float32)
        k, p, mp = int(rng.integers(0, V + 2)), float(rng.uniform(0.01, 1.0)), float(rng.uniform(0, 1))
        d = oracle.support_row(s, k, p, mp)
        mask = oracle.in_support(s, d["key_thr"], d["id_thr"])
        assert mask.sum() == d["n"] >= 1
        assert mask[int(np.argmax(s))]                            # lowest-id argmax kept
        assert set(np.nonzero(mask)[0]) == set(d["pi"][: d["n"]])  # a prefix of the order
        e = np.exp(s.astype(np.float64) - s.max())
        assert abs((e * mask).sum() / (e * mask).sum() - 1.0) < 1e-12
        q = np.where(mask, e, 0) / (e * mask).sum()
        assert abs(q.sum() - 1.0) < 1e-12


# ---------------------------------------------------------------- values
def _problem(rng, T=6, H=16, V=40, scale=1.0):
    h = rng.standard_normal((T, H)).astype(np.float32)
    W = (rng.standard_normal((V, H)) * 0.3 * scale).astype(np.float32)
    temp = rng.uniform(0.5, 1.5, T).astype(np.float32)
    return h, W, temp


def test_identity_rows_equal_log_softmax(rng):
    from scipy.special import log_softmax
    h, W, temp = _problem(rng, T=8, V=50)
    y = rng.integers(0, 50, 8)
    f = oracle.forward(h, W, y, temp)
    z = h.astype(np.float64) @ W.astype(np.float64).T
    ref = log_softmax(z / temp.astype(np.float64)[:, None], axis=1)[np.arange(8), y]
    np.testing.assert_allclose(f["logprob"], np.minimum(ref, 0), rtol=0, atol=1e-13)
    assert np.all(f["n"] == 50)


def test_filtered_logprob_closed_form():
    # z/T = [3, 1, 1, 0, -2] with T = 1, top-k 2 keeps ids {0, 1}
    s = np.array([3.0, 1.0, 1.0, 0.0, -2.0])
    h = np.ones((1, 1), np.float32)
    W = s[:, None].astype(np.float32)
    f = oracle.forward(h, W, np.array([1]), top_k=np.array([2]))
    assert f["n"][0] == 2 and f["id_thr"][0] == 1
    assert abs(f["logprob"][0] - (-math.log1p(math.exp(2.0)))) < 1e-14
    # target 2 ties target 1 but loses the id tie-break: out of support
    f = oracle.forward(h, W, np.array([2]), top_k=np.array([2]))
    assert f["logprob"][0] == -math.inf and not f["in_support"][0]
    # temperature 2 then min-p 0.5: keep s/T - max >= ln 0.5, i.e. z >= 3 - 2 ln 2 = 1.61
    f = oracle.forward(h, W, np.array([0]), np.array([2.0], np.float32), min_p=np.array([0.5]))
    assert f["n"][0] == 1 and f["logprob"][0] == 0.0


def test_out_of_support_has_minus_inf_and_zero_gradient(rng):
    h, W, temp = _problem(rng, T=4, V=30, scale=3)
    f0 = oracle.forward(h, W, np.zeros(4, np.int64), temp, top_k=np.full(4, 3))
    order = [oracle.order_row(f0["keys"][t]) for t in range(4)]
    y = np.array([order[t][-1] for t in range(4)])             # last token: never in a top-3
    f = oracle.forward(h, W, y, temp, top_k=np.full(4, 3))
    assert np.all(f["logprob"] == -np.inf)
    dH, dW = oracle.backward(h, W, y, f, np.full(4, 7.0), temp)
    assert not dH.any() and not dW.any()


def test_logprob_is_clamped_nonpositive(rng):
    h, W, temp = _problem(rng, T=10, V=20, scale=4)
    f = oracle.forward(h, W, rng.integers(0, 20, 10), temp, top_k=np.ones(10, np.int64))
    assert np.all((f["logprob"] <= 0) | np.isinf(f["logprob"]))


# ---------------------------------------------------------------- gradients
def _loss(h, W, y, temp, meta, g, support_of):
    """sum_t g_t logprob_t with each row's support frozen to ``support_of``."""
    z = h @ W.T
    u = z / temp[:, None]
    tot = 0.0
    for t in range(len(y)):
        S = support_of[t]
        mx = u[t, S].max()
        tot += g[t] * (u[t, y[t]] - (mx + math.log(np.exp(u[t, S] - mx).sum())))
    return tot


def test_gradients_match_central_differences(rng):
    T, H, V = 4, 8, 12
    h, W, temp = _problem(rng, T, H, V, scale=2)
    meta = dict(top_k=np.array([0, 5, 0, 3]), top_p=np.array([1.0, 1.0, 0.8, 0.9], np.float32),
                min_p=np.array([0.0, 0.0, 0.0, 0.05], np.float32))
    f0 = oracle.forward(h, W, np.zeros(T, np.int64), temp, **meta)
    y = np.array([f0["keys"][t].argmax() for t in range(T)])
    f = oracle.forward(h, W, y, temp, **meta)
    assert f["in_support"].all()
    S = [oracle.order_row(f["keys"][t])[: f["n"][t]] for t in range(T)]
    g = rng.standard_normal(T)
    dH, dW = oracle.backward(h, W, y, f, g, temp)
    h64, W64, t64 = h.astype(np.float64), W.astype(np.float64), temp.astype(np.float64)
    eps = 1e-6
    for (arr, grad) in ((h64, dH), (W64, dW)):
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            old = arr[idx]
            arr[idx] = old + eps
            fp = _loss(h64, W64, y, t64, meta, g, S)
            arr[idx] = old - eps
            fm = _loss(h64, W64, y, t64, meta, g, S)
            arr[idx] = old
            num[idx] = (fp - fm) / (2 * eps)
        rel = np.linalg.norm(num - grad) / np.linalg.norm(grad)
        assert rel < 1e-6, rel
    # the supports did not move under the perturbation size used
    for d in (+eps, -eps):
        fz = oracle.forward(h + d, W, y, temp, **meta)
        assert np.array_equal(fz["n"], f["n"])


def test_gradients_match_torch_autograd(rng):
    torch = pytest.importorskip("torch")
    T, H, V = 5, 12, 30
    h, W, temp = _problem(rng, T, H, V, scale=2)
    meta = dict(top_k=np.array([0, 4, 0, 0, 7]), top_p=np.array([1.0, 1.0, 0.7, 1.0, 0.95], np.float32),
                min_p=np.array([0.0, 0.0, 0.0, 0.2, 0.0], np.float32))
    f0 = oracle.forward(h, W, np.zeros(T, np.int64), temp, **meta)
    y = np.array([oracle.order_row(f0["keys"][t])[0] for t in range(T)])
    f = oracle.forward(h, W, y, temp, **meta)
    g = rng.standard_normal(T)
    dH, dW = oracle.backward(h, W, y, f, g, temp)
    th = torch.tensor(h, dtype=torch.float64, requires_grad=True)
    tW = torch.tensor(W, dtype=torch.float64, requires_grad=True)
    u = (th @ tW.T) / torch.tensor(temp, dtype=torch.float64)[:, None]
    L = 0
    for t in range(T):
        S = torch.tensor(oracle.order_row(f["keys"][t])[: f["n"][t]])
        L = L + float(g[t]) * (u[t, int(y[t])] - torch.logsumexp(u[t, S], 0))
    L.backward()
    np.testing.assert_allclose(dH, th.grad.numpy(), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(dW, tW.grad.numpy(), rtol=1e-12, atol=1e-14)


def test_loss_sign_convention(rng):
    """The descent direction of the NLL is (q - onehot)/T = -d logprob/dz."""
    torch = pytest.importorskip("torch")
    h, W, temp = _problem(rng, 1, 6, 11)
    y = np.array([3])
    f = oracle.forward(h, W, y, temp)
    dz = oracle.dlogits(h, W, y, f, np.array([1.0]), temp)
    z = torch.tensor(h.astype(np.float64) @ W.astype(np.float64).T, requires_grad=True)
    nll = -torch.log_softmax(z / float(temp[0]), 1)[0, 3]
    nll.backward()
    np.testing.assert_allclose(-dz, z.grad.numpy(), atol=1e-15)


def test_weight_gradient_columns_sum_to_zero(rng):
    h, W, temp = _problem(rng, T=6, V=25, scale=2)
    f = oracle.forward(h, W, np.zeros(6, np.int64), temp, top_p=np.full(6, 0.9, np.float32))
    dH, dW = oracle.backward(h, W, np.zeros(6, np.int64), f, rng.standard_normal(6), temp)
    assert np.abs(dW.sum(axis=0)).max() < 1e-12 * max(1.0, np.abs(dW).max())


def test_gradient_products_take_sparse_dz_with_the_same_sums():
    """dz is nonzero only on the support; the products dz W and dz^T h of a
    scipy.sparse copy equal the dense ones (pins the sparse form a full-size
    test uses), and equal a hand loop over the nonzeros.  (Its own generator:
    the session one feeds the pins that follow.)"""
    sp = pytest.importorskip("scipy.sparse")
    rng = np.random.Generator(np.random.PCG64(515))
    h, W, temp = _problem(rng, T=7, V=40, scale=2)
    meta = dict(top_k=np.array([3, 0, 5, 1, 0, 2, 4]), top_p=np.array([1, .8, 1, 1, .6, 1, 1], np.float32))
    y = np.array([oracle.order_row(oracle.forward(h, W, np.zeros(7, np.int64), temp, **meta)["keys"][t])[0]
                  for t in range(7)])
    f = oracle.forward(h, W, y, temp, **meta)
    g = rng.standard_normal(7)
    dz = oracle.dlogits(h, W, y, f, g, temp)
    dH, dW = oracle.backward(h, W, y, f, g, temp)
    sH, sW = oracle.gradient_products(sp.csr_matrix(dz), h, W)
    np.testing.assert_allclose(sH, dH, rtol=1e-14, atol=1e-16)
    np.testing.assert_allclose(sW, dW, rtol=1e-14, atol=1e-16)
    loopW = np.zeros_like(dW)
    for t, j in zip(*np.nonzero(dz)):
        loopW[j] += dz[t, j] * h[t].astype(np.float64)
    np.testing.assert_allclose(loopW, dW, rtol=1e-13, atol=1e-16)
    assert (np.count_nonzero(dz, axis=1) <= np.where(meta["top_k"] > 0, meta["top_k"], 40)).all()


def test_sampled_targets_lie_in_support(rng):
    h, W, temp = _problem(rng, T=30, V=64, scale=3)
    meta = dict(top_k=rng.choice([0, 5], 30), top_p=rng.choice([1.0, 0.7], 30).astype(np.float32),
                min_p=rng.choice([0.0, 0.1], 30).astype(np.float32))
    y = oracle.sample_targets(h, W, temp, meta["top_k"], meta["top_p"], meta["min_p"], rng.random(30))
    f = oracle.forward(h, W, y, temp, **meta)
    assert f["in_support"].all()


def test_bad_metadata_is_rejected():
    s = np.zeros(4, np.float32)
    for args in ((-1, 1.0, 0.0), (0, 0.0, 0.0), (0, 1.5, 0.0), (0, 1.0, -0.1), (0, 1.0, 1.5)):
        with pytest.raises(ValueError):
            oracle.support_row(s, *args)
    with pytest.raises(ValueError):
        oracle.forward(np.ones((1, 2), np.float32), np.ones((3, 2), np.float32), np.array([0]),
                       np.array([0.0], np.float32))


# ---------------------------------------------------------------- policy-gradient loss
def _pg_problem(rng, T=6, H=10, V=24):
    h, W, temp = _problem(rng, T, H, V, scale=2)
    meta = dict(top_k=np.array([0, 5, 0, 8, 0, 3][:T]), top_p=np.array([1.0, 1.0, 0.9, 1.0, 0.8, 1.0][:T], np.float32),
                min_p=np.zeros(T, np.float32))
    f0 = oracle.forward(h, W, np.zeros(T, np.int64), temp, **meta)
    y = np.array([oracle.order_row(f0["keys"][t])[t % 2] for t in range(T)])
    f = oracle.forward(h, W, y, temp, **meta)
    assert f["in_support"].all()
    # old logprobs put the ratios on both sides of both clip bounds
    offs = np.array([-1.0, -0.1, 0.05, 0.4, 1.3, -0.6][:T])
    old = (f["logprob"] + offs).astype(np.float32)
    A = np.array([1.5, -0.7, 2.0, -1.2, 0.8, -2.5][:T], np.float32)
    return h, W, temp, meta, y, f, old, A


@pytest.mark.parametrize("objective", ["cispo", "clip"])
def test_policy_gradient_matches_autograd_of_objective(rng, objective):
    """d loss / d(h, W) through the selected logprob, against fp64 autograd of
    the objective written on the logits (CISPO's weight detached)."""
    torch = pytest.importorskip("torch")
    h, W, temp, meta, y, f, old, A = _pg_problem(rng)
    el, eh, sc = (float(np.float32(x)) for x in (0.2, 0.28, 0.125))   # parameters are fp32 values
    pg = oracle.policy_loss(f["logprob"], A, old, objective, el, eh, sc)
    dH, dW = oracle.backward(h, W, y, f, pg["g"], temp)
    th = torch.tensor(h, dtype=torch.float64, requires_grad=True)
    tW = torch.tensor(W, dtype=torch.float64, requires_grad=True)
    u = (th @ tW.T) / torch.tensor(temp, dtype=torch.float64)[:, None]
    L = 0
    for t in range(len(y)):
        S = torch.tensor(oracle.order_row(f["keys"][t])[: f["n"][t]])
        lp = torch.clamp(u[t, int(y[t])] - torch.logsumexp(u[t, S], 0), max=0.0)
        r = torch.exp(lp - float(old[t]))
        a = float(A[t])
        if objective == "cispo":
            L = L - a * torch.clamp(r, max=1 + eh).detach() * lp
        else:
            L = L - torch.minimum(r * a, torch.clamp(r, 1 - el, 1 + eh) * a)
    L = L * sc
    L.backward()
    assert abs(float(L) - pg["loss"].sum()) < 1e-12 * max(1.0, abs(float(L)))
    np.testing.assert_allclose(dH, th.grad.numpy(), rtol=1e-11, atol=1e-14)
    np.testing.assert_allclose(dW, tW.grad.numpy(), rtol=1e-11, atol=1e-14)


def test_policy_loss_special_cases():
    """Hand-worked values: ratio 1, zero advantage, each clip branch, -inf and NaN rows."""
    e = math.e
    lp = np.array([-0.5, -0.5, -1.0, -1.0, -2.0, -1.0, -3.0, -math.inf, math.nan])
    # ratio:        1     1     e     e^-1  e     e^-1   1     -       -
    old = np.array([-0.5, -0.5, -2.0, 0.0, -3.0, 0.0, -3.0, -1.0, -1.0], np.float32)
    A = np.array([2.0, 0.0, 2.0, -2.0, -2.0, 2.0, -1.0, 3.0, 3.0], np.float32)
    c = oracle.policy_loss(lp, A, old, "clip", eps_low=0.25, eps_high=0.5)
    want_loss = [2.0 * -1, 0.0, -1.5 * 2.0, 0.75 * 2.0, 2.0 * e, -2.0 / e, 1.0, 0.0, math.nan]
    want_g = [-2.0, 0.0, 0.0, 0.0, 2.0 * e, -2.0 / e, 1.0, 0.0, 0.0]
    np.testing.assert_allclose(c["loss"], want_loss, rtol=1e-6)
    np.testing.assert_allclose(c["g"], want_g, rtol=1e-6, atol=1e-12)
    k = oracle.policy_loss(lp, A, old, "cispo", eps_high=0.5)
    # weight min(r, 1.5): 1, 1, 1.5, e^-1, 1.5, e^-1, 1
    w = [1.0, 1.0, 1.5, 1 / e, 1.5, 1 / e, 1.0]
    want_g = [-A[i] * w[i] for i in range(7)] + [0.0, 0.0]
    want_loss = [-A[i] * w[i] * lp[i] for i in range(7)] + [0.0, math.nan]
    np.testing.assert_allclose(k["loss"], want_loss, rtol=1e-6, atol=1e-12)
    np.testing.assert_allclose(k["g"], want_g, rtol=1e-6, atol=1e-12)
    s = oracle.policy_loss(lp[:1], A[:1], old[:1], "cispo", scale=0.25)
    assert s["loss"][0] == 0.25 * -2.0 * -0.5 * 1.0 and s["g"][0] == 0.25 * -2.0
    with pytest.raises(ValueError):
        oracle.policy_loss(lp, A, old, "ppo")


def test_clipped_policy_gradient_matches_central_differences(rng):
    """The clipped surrogate has a true gradient away from its kinks."""
    h, W, temp, meta, y, f, old, A = _pg_problem(rng, T=4, H=6, V=10)
    S = [oracle.order_row(f["keys"][t])[: f["n"][t]] for t in range(4)]
    el, eh = float(np.float32(0.2)), float(np.float32(0.28))
    pg = oracle.policy_loss(f["logprob"], A, old, "clip", el, eh)
    dH, dW = oracle.backward(h, W, y, f, pg["g"], temp)
    h64, W64, t64 = h.astype(np.float64), W.astype(np.float64), temp.astype(np.float64)

    def total(hh, WW):
        u = (hh @ WW.T) / t64[:, None]
        tot = 0.0
        for t in range(4):
            mx = u[t, S[t]].max()
            lp = min(u[t, y[t]] - (mx + math.log(np.exp(u[t, S[t]] - mx).sum())), 0.0)
            r = math.exp(lp - float(old[t]))
            tot += -min(r * float(A[t]), min(max(r, 1 - el), 1 + eh) * float(A[t]))
        return tot

    eps = 1e-6
    for arr, grad in ((h64, dH), (W64, dW)):
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            o = arr[idx]
            arr[idx] = o + eps
            fp = total(h64, W64)
            arr[idx] = o - eps
            fm = total(h64, W64)
            arr[idx] = o
            num[idx] = (fp - fm) / (2 * eps)
        rel = np.linalg.norm(num - grad) / np.linalg.norm(grad)
        assert rel < 1e-6, rel


# ---------------------------------------------------------------- side outputs: entropies, full LSE
def test_entropy_closed_forms():
    # all-equal logits: log V over the row; top-k 7 keeps 7 tokens (ties split by id): log 7
    V = 50
    h = np.ones((1, 1), np.float32)
    W = np.zeros((V, 1), np.float32)
    f = oracle.forward(h, W, np.array([0]), top_k=np.array([7]))
    assert abs(f["entropy_full"][0] - math.log(V)) < 1e-13
    assert abs(f["entropy_support"][0] - math.log(7)) < 1e-13
    assert abs(f["lse_full"][0] - math.log(V)) < 1e-13
    # top-k 1: a one-token support has zero entropy
    W = np.arange(V, dtype=np.float32)[:, None] * 0.1
    f = oracle.forward(h, W, np.array([V - 1]), top_k=np.array([1]))
    assert f["entropy_support"][0] == 0.0
    # two tokens a bit apart, temperature 0.5: binary entropy of sigmoid(2 d)
    W = np.array([[1.0], [0.25], [-3.0]], np.float32)
    f = oracle.forward(h, W, np.array([0]), np.array([0.5], np.float32), top_k=np.array([2]))
    q = 1.0 / (1.0 + math.exp(-2 * 0.75))
    assert abs(f["entropy_support"][0] - (-q * math.log(q) - (1 - q) * math.log(1 - q))) < 1e-13


def test_entropy_matches_scipy_and_bounds(rng):
    from scipy.special import softmax
    from scipy.stats import entropy
    h, W, temp = _problem(rng, T=8, V=60, scale=3)
    meta = dict(top_k=rng.choice([0, 5, 20], 8), top_p=rng.choice([1.0, 0.6], 8).astype(np.float32),
                min_p=rng.choice([0.0, 0.1], 8).astype(np.float32))
    f = oracle.forward(h, W, np.zeros(8, np.int64), temp, **meta)
    u = (h.astype(np.float64) @ W.astype(np.float64).T) / temp.astype(np.float64)[:, None]
    for t in range(8):
        S = oracle.order_row(f["keys"][t])[: f["n"][t]]
        assert abs(f["entropy_full"][t] - entropy(softmax(u[t]))) < 1e-12
        assert abs(f["entropy_support"][t] - entropy(softmax(u[t, S]))) < 1e-12
        assert -1e-15 <= f["entropy_support"][t] <= math.log(f["n"][t]) + 1e-12
        assert f["entropy_full"][t] <= math.log(60) + 1e-12
        assert abs(f["lse_full"][t] - (u[t].max() + math.log(np.exp(u[t] - u[t].max()).sum()))) < 1e-12


# ---------------------------------------------------------------- ignore_index rows
def test_ignored_rows_score_zero_and_get_no_gradient(rng):
    h, W, temp = _problem(rng, T=6, V=30, scale=2)
    y = np.array([3, -100, 7, -100, 0, 11])
    meta = dict(top_k=np.array([0, 4, 0, 0, 5, 0]), top_p=np.full(6, 0.9, np.float32))
    f = oracle.forward(h, W, y, temp, **meta, ignore_index=-100)
    assert list(f["ignored"]) == [False, True, False, True, False, False]
    assert f["logprob"][1] == 0.0 and f["logprob"][3] == 0.0
    # the active rows are scored exactly as without the ignored ones
    act = np.array([0, 2, 4, 5])
    g = oracle.forward(h, W, y, temp, **meta, rows=act)
    assert np.array_equal(f["logprob"][act], g["logprob"])
    # ignored rows still have a support and side outputs
    assert f["n"][1] == 4 and np.isfinite(f["entropy_support"][[1, 3]]).all()
    dH, dW = oracle.backward(h, W, y, f, np.ones(6), temp)
    assert not dH[[1, 3]].any()
    dH2, dW2 = oracle.backward(h, W, y, g, np.ones(6), temp)
    np.testing.assert_allclose(dW, dW2, rtol=0, atol=0)          # ignored rows add nothing to dW
    with pytest.raises(AssertionError):
        oracle.forward(h, W, y, temp, ignore_index=None)         # -100 is not a token without ignore_index


# ---------------------------------------------------------------- scalar pre-GEMM temperature
def test_round_to_bf16_matches_torch_and_ties_to_even(rng):
    torch = pytest.importorskip("torch")
    mag = np.float32(10.0) ** rng.integers(-30, 30, 20000).astype(np.float32)
    x = np.concatenate([rng.standard_normal(20000).astype(np.float32) * mag,
                        np.float32([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 1 + 2 ** -8 + 2 ** -20, 0.0, -0.0])])
    x = x[np.isfinite(x)]
    ref = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    assert np.array_equal(oracle.round_to_bf16(x).view(np.uint32), ref.view(np.uint32))
    assert oracle.round_to_bf16(np.float32([1 + 2 ** -8]))[0] == 1.0              # tie, down to even
    assert oracle.round_to_bf16(np.float32([1 + 3 * 2 ** -8]))[0] == 1 + 2 ** -6   # tie, up to even


def test_pre_gemm_hidden_matches_torch_division_and_rounding(rng):
    torch = pytest.importorskip("torch")
    h = rng.standard_normal((7, 33)).astype(np.float32) * 3
    for t in (0.7, 1.3, 0.05):
        ref = (torch.from_numpy(h) / torch.tensor(t, dtype=torch.float32)).to(torch.bfloat16).float().numpy()
        assert np.array_equal(oracle.pre_gemm_hidden(h, t, "bf16").view(np.uint32), ref.view(np.uint32))
        ref32 = (torch.from_numpy(h) / torch.tensor(t, dtype=torch.float32)).numpy()
        assert np.array_equal(oracle.pre_gemm_hidden(h, t, "f32").view(np.uint32), ref32.view(np.uint32))
    assert np.array_equal(oracle.pre_gemm_hidden(h, 1.0, "f32"), h)


def _pre_gemm_case(rng, Tn=12, H=16, V=40):
    h = oracle.round_to_bf16(rng.standard_normal((Tn, H)).astype(np.float32))
    W = oracle.round_to_bf16((rng.standard_normal((V, H)) * 0.3).astype(np.float32))
    z = h.astype(np.float64) @ W.astype(np.float64).T
    y = np.where(np.arange(Tn) % 3 == 0, rng.integers(0, V, Tn), z.argmax(1)).astype(np.int64)
    tk = np.where(np.arange(Tn) % 2 == 0, 8, 0).astype(np.int32)
    tp = np.where(np.arange(Tn) % 4 == 1, 0.9, 1.0).astype(np.float32)
    mp = np.where(np.arange(Tn) % 5 == 2, 0.05, 0.0).astype(np.float32)
    return h, W, y, tk, tp, mp


def test_pre_gemm_temperature_equals_post_gemm_for_a_power_of_two(rng):
    """T = 0.5 divides exactly (h / T = 2h in bf16, fl32(z) / T = 2 fl32(z)),
    so the scalar pre-GEMM convention gives the post-GEMM convention's keys,
    logprobs and gradients, row by row."""
    h, W, y, tk, tp, mp = _pre_gemm_case(rng)
    Tn = h.shape[0]
    hs = oracle.pre_gemm_hidden(h, 0.5, "bf16")
    assert np.array_equal(hs, 2 * h)
    t = np.full(Tn, 0.5, np.float32)
    post = oracle.forward(h, W, y, t, tk, tp, mp)
    pre = oracle.forward(hs, W, y, None, tk, tp, mp)
    assert np.array_equal(pre["keys"].view(np.uint32), post["keys"].view(np.uint32))
    assert np.array_equal(pre["logprob"], post["logprob"]) and pre["in_support"].any()
    g = rng.standard_normal(Tn)
    dh1, dw1 = oracle.backward(h, W, y, post, g, t)
    dh2, dw2 = oracle.backward_pre_gemm(hs, W, y, pre, g, 0.5)
    np.testing.assert_allclose(dh2, dh1, rtol=1e-13, atol=1e-300)
    np.testing.assert_allclose(dw2, dw1, rtol=1e-13, atol=1e-300)


def test_pre_gemm_gradient_matches_autograd(rng):
    """fp64 autograd of sum_r g_r (u[r, y_r] - logsumexp of u[r] over the
    support), u = (h / T) W^T, for T = 0.7 (the pre-GEMM quotient unrounded
    here: the oracle's fp32 rounding of h / T accounts for ~1e-7)."""
    torch = pytest.importorskip("torch")
    h, W, y, tk, _, _ = _pre_gemm_case(rng, Tn=6, H=10, V=30)
    y = (h.astype(np.float64) @ W.astype(np.float64).T).argmax(1)   # all targets in support
    t = 0.7
    hs = oracle.pre_gemm_hidden(h, t, "f32")
    fwd = oracle.forward(hs, W, y, None, tk, None, None)
    assert fwd["in_support"].all()
    g = rng.standard_normal(h.shape[0])
    dH, dW = oracle.backward_pre_gemm(hs, W, y, fwd, g, t)
    H64 = torch.tensor(h.astype(np.float64), requires_grad=True)
    W64 = torch.tensor(W.astype(np.float64), requires_grad=True)
    u = (H64 / t) @ W64.T
    total = 0
    for r in range(h.shape[0]):
        mask = torch.tensor(oracle.in_support(fwd["keys"][r], int(fwd["key_thr"][r]), int(fwd["id_thr"][r])))
        total = total + float(g[r]) * (u[r, int(y[r])] - torch.logsumexp(u[r][mask], 0))
    total.backward()
    for a, b in ((dH, H64.grad.numpy()), (dW, W64.grad.numpy())):
        assert np.linalg.norm(a - b) / np.linalg.norm(b) < 1e-6


# ---------------------------------------------------------------- bf16 value lane
def _bf16_round_exact(q: Fraction) -> Fraction:
    """An exact rational rounded to 8 significant bits, nearest with ties to
    even (normal range), in exact arithmetic."""
    if q == 0:
        return Fraction(0)
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    ulp = Fraction(2) ** (e - 7)
    m = a / ulp                                   # in [128, 256)
    n = m.numerator // m.denominator
    r = m - n
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return (n * ulp) if q > 0 else -(n * ulp)


def _lane_problem(rng, T=6, H=16, V=40):
    h = oracle.round_to_bf16(rng.standard_normal((T, H)).astype(np.float32) * 2)
    W = oracle.round_to_bf16(rng.standard_normal((V, H)).astype(np.float32))
    temp = rng.uniform(0.1, 3.0, T).astype(np.float32)
    return h, W, temp


def test_bf16_lane_keys_follow_the_value_program_exactly(rng):
    """Each key is bf16(fl32(bf16(fl32(z)) / T)), every step an exact
    rational rounding; keys are bf16 values."""
    h, W, temp = _lane_problem(rng)
    z64 = h.astype(np.float64) @ W.astype(np.float64).T
    s = oracle.bf16_lane_keys(z64, temp)
    assert np.all((s.view(np.uint32) & 0xFFFF) == 0)
    for t in range(h.shape[0]):
        for j in range(W.shape[0]):
            z = sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(h[t], W[j]))
            zb = _bf16_round_exact(Fraction(float(_f32_round_exact(z))))
            q = _f32_round_exact(zb / Fraction(float(temp[t])))
            want = _bf16_round_exact(Fraction(float(q)))
            assert Fraction(float(s[t, j])) == want, (t, j)
    # small integer logits at T = 1 are bf16 values: the keys are the logits
    hi = np.float32(rng.integers(-3, 4, (4, 8)))
    Wi = np.float32(rng.integers(-3, 4, (10, 8)))
    zi = hi.astype(np.float64) @ Wi.astype(np.float64).T
    assert np.array_equal(oracle.bf16_lane_keys(zi, np.ones(4, np.float32)), zi.astype(np.float32) + 0)


def test_bf16_lane_logprob_is_the_bf16_log_softmax_of_the_keys(rng):
    torch = pytest.importorskip("torch")
    from scipy.special import log_softmax
    h, W, temp = _lane_problem(rng, T=8, V=50)
    y = rng.integers(0, 50, 8)
    f = oracle.forward(h, W, y, temp, lane="bf16")
    ref = np.minimum(log_softmax(f["keys"].astype(np.float64), axis=1)[np.arange(8), y], 0)
    want = torch.from_numpy(ref).float().bfloat16().double().numpy()
    assert np.array_equal(f["logprob"], want)
    # top-k 1 keeps the lowest-id maximum only: logprob exactly 0
    yk = np.array([oracle.order_row(f["keys"][t])[0] for t in range(8)])
    fk = oracle.forward(h, W, yk, temp, top_k=np.ones(8, np.int32), lane="bf16")
    assert np.all(fk["logprob"] == 0.0)


def test_bf16_lane_gradient_is_the_straight_through_vjp(rng):
    """fp64 autograd of sum_r g_r (u[r, y_r] - logsumexp of u[r] over the
    support), u = z / T carrying the bf16 keys' values (the roundings pass
    gradients unchanged)."""
    torch = pytest.importorskip("torch")
    T, V = 5, 30
    h, W, temp = _lane_problem(rng, T=T, V=V)
    meta = dict(top_k=np.array([0, 4, 0, 0, 7]), top_p=np.array([1.0, 1.0, 0.7, 1.0, 0.95], np.float32),
                min_p=np.array([0.0, 0.0, 0.0, 0.2, 0.0], np.float32))
    f0 = oracle.forward(h, W, np.zeros(T, np.int64), temp, **meta, lane="bf16")
    y = np.array([oracle.order_row(f0["keys"][t])[0] for t in range(T)])
    f = oracle.forward(h, W, y, temp, **meta, lane="bf16")
    assert f["in_support"].all()
    g = rng.standard_normal(T)
    dH, dW = oracle.backward(h, W, y, f, g, temp)
    th = torch.tensor(h, dtype=torch.float64, requires_grad=True)
    tW = torch.tensor(W, dtype=torch.float64, requires_grad=True)
    zt = (th @ tW.T) / torch.tensor(temp, dtype=torch.float64)[:, None]
    u = zt + (torch.tensor(f["keys"], dtype=torch.float64) - zt).detach()
    L = 0
    for t in range(T):
        S = torch.tensor(oracle.order_row(f["keys"][t])[: f["n"][t]])
        L = L + float(g[t]) * (u[t, int(y[t])] - torch.logsumexp(u[t, S], 0))
    L.backward()
    np.testing.assert_allclose(dH, th.grad.numpy(), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(dW, tW.grad.numpy(), rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------- fp8 lane
def test_e4m3_encode_matches_torch_and_ties_to_even():
    """The encoder against torch's float8_e4m3fn cast (round to nearest,
    ties to even) over every magnitude of the format, subnormals, exact ties
    and the largest finite value; decode(encode(x)) is that cast's value."""
    torch = pytest.importorskip("torch")
    rng = np.random.Generator(np.random.PCG64(88))
    mag = np.exp2(rng.uniform(-12, np.log2(448.0), 40000))
    x = (mag * rng.choice([-1.0, 1.0], mag.size)).astype(np.float32)
    x = np.clip(x, -448, 448).astype(np.float32)
    vals = oracle.e4m3_decode(np.arange(256, dtype=np.uint8)[(np.arange(256) & 0x7F) != 0x7F])
    pos = np.unique(np.abs(vals))
    mids = ((pos[1:] + pos[:-1]) / 2).astype(np.float32)              # exact ties between neighbours
    x = np.concatenate([x, mids, -mids, np.float32([0.0, -0.0, 448.0, -448.0, 2.0 ** -9, 2.0 ** -10, 1.0625])])
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn)
    assert np.array_equal(oracle.e4m3_encode(x), ref.view(torch.uint8).numpy())
    assert np.array_equal(oracle.e4m3_decode(oracle.e4m3_encode(x)), ref.float().numpy().astype(np.float64))
    assert oracle.e4m3_encode(np.float32([1.0625]))[0] == 0x38                   # tie down to even (1.0)
    assert oracle.e4m3_encode(np.float32([1.1875]))[0] == 0x3A                   # tie up to even (1.25)


def test_e4m3_decode_is_the_format_on_every_code():
    torch = pytest.importorskip("torch")
    codes = np.arange(256, dtype=np.uint8)
    codes = codes[(codes & 0x7F) != 0x7F]                              # the two NaN codes excluded
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()
    assert np.array_equal(oracle.e4m3_decode(codes), ref.astype(np.float64))
    assert oracle.e4m3_decode(np.uint8([0x7E]))[0] == 448.0 and oracle.e4m3_decode(np.uint8([0x01]))[0] == 2.0 ** -9


def test_fp8_row_quantization_closed_forms():
    """The row maximum maps to +-448 exactly; a zero row keeps scale 1 and
    zero codes; every value lies within half an e4m3 step of its code times
    the scale."""
    rng = np.random.Generator(np.random.PCG64(89))
    h = (rng.standard_normal((6, 40)) * rng.uniform(0.01, 50, (6, 1))).astype(np.float32)
    h[3] = 0.0
    codes, a = oracle.fp8_quantize_rows(h)
    amax = np.abs(h).max(1)
    for t in range(6):
        if t == 3:
            assert a[t] == 1.0 and not codes[t].any()
            continue
        assert a[t] == np.float32(amax[t] / np.float32(448.0))
        k = int(np.argmax(np.abs(h[t])))
        assert oracle.e4m3_decode(codes[t, k:k + 1])[0] == np.copysign(448.0, h[t, k])
    deq = oracle.fp8_dequant_rows(h).astype(np.float64)
    step = np.maximum(np.exp2(np.floor(np.log2(np.maximum(np.abs(h) / a[:, None], 2.0 ** -6))) - 3), 2.0 ** -9)
    assert np.all(np.abs(deq - h) <= 0.5 * step * a[:, None] * (1 + 1e-6) + 1e-30)


def test_fp8_logits_reduce_to_the_plain_product_on_exact_operands():
    """Hidden rows whose values are e4m3 values times a power of two with the
    row maximum 448 times it quantize exactly, and a power-of-two weight
    scale dequantizes exactly: the fp8 lane's logits are then h W_deq^T."""
    rng = np.random.Generator(np.random.PCG64(90))
    pos = np.unique(np.abs(oracle.e4m3_decode(np.arange(0x7F, dtype=np.uint8))))
    hv = rng.choice(pos, (5, 32)) * rng.choice([-1, 1], (5, 32))
    hv[:, 0] = 448.0
    h = (hv * np.exp2(rng.integers(-4, 3, (5, 1)))).astype(np.float32)
    w8 = rng.integers(0, 0x7E, (9, 32)).astype(np.uint8) | (rng.integers(0, 2, (9, 32)) << 7).astype(np.uint8)
    w_scale = np.exp2(rng.integers(-8, -2, 9)).astype(np.float32)
    assert np.array_equal(oracle.fp8_dequant_rows(h), h.astype(np.float64))
    z = oracle.fp8_logits(h, w8, w_scale)
    ref = h.astype(np.float64) @ oracle.fp8_dequant_weight(w8, w_scale).T
    np.testing.assert_allclose(z, ref, rtol=1e-15, atol=0)


def test_fp8_lane_gradient_is_the_straight_through_vjp():
    """fp64 autograd of the selected logprob with the product's operands
    taken as the dequantized values (quantization passes gradients
    unchanged): dH = dz W_deq, dW = dz^T h_deq."""
    torch = pytest.importorskip("torch")
    rng = np.random.Generator(np.random.PCG64(91))
    T, H, V = 4, 16, 30
    h = rng.standard_normal((T, H)).astype(np.float32)
    w8 = (rng.integers(0x20, 0x50, (V, H)) | (rng.integers(0, 2, (V, H)) << 7)).astype(np.uint8)
    w_scale = rng.uniform(0.01, 0.05, V).astype(np.float32)
    temp = rng.uniform(0.6, 1.4, T).astype(np.float32)
    meta = dict(top_k=np.array([0, 5, 0, 7]), top_p=np.array([1.0, 1.0, 0.8, 1.0], np.float32))
    f0 = oracle.forward(h, w8, np.zeros(T, np.int64), temp, **meta, lane="fp8", w_scale=w_scale)
    y = np.array([oracle.order_row(f0["keys"][t])[1] for t in range(T)])
    f = oracle.forward(h, w8, y, temp, **meta, lane="fp8", w_scale=w_scale)
    assert f["in_support"].all()
    g = rng.standard_normal(T)
    dH, dW = oracle.backward(h, w8, y, f, g, temp, w_scale=w_scale)
    hq = torch.tensor(oracle.fp8_dequant_rows(h), requires_grad=True)
    wq = torch.tensor(oracle.fp8_dequant_weight(w8, w_scale), requires_grad=True)
    # the lane's logits from the dequantized operands: h_deq W_deq^T = (h8 W8^T) sW a
    u = (hq @ wq.T) / torch.tensor(temp.astype(np.float64))[:, None]
    loss = 0.0
    for t in range(T):
        mask = torch.tensor(oracle.in_support(f["keys"][t], int(f["key_thr"][t]), int(f["id_thr"][t])))
        loss = loss + float(g[t]) * (u[t, y[t]] - torch.logsumexp(u[t][mask], 0))
    loss.backward()
    np.testing.assert_allclose(dH, hq.grad.numpy(), rtol=1e-10, atol=1e-14)
    np.testing.assert_allclose(dW, wq.grad.numpy(), rtol=1e-10, atol=1e-14)
    np.testing.assert_allclose(oracle.fp8_logits(h, w8, w_scale),
                               (hq @ wq.T).detach().numpy(), rtol=1e-13, atol=1e-15)
