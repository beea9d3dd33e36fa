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
import multiprocessing

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import GRAD_RTOL, LOGPROB_ATOL, dev, meta_of, rel_fro, say, to_gpu
from sampling_transform_logprob_amd import binding, workloads

pytestmark = pytest.mark.gpu

_CACHE = {}


def _workload(name):
    """Full-size inputs, drawn once per module (the weight draw takes tens of
    seconds at these sizes)."""
    if name not in _CACHE:
        _CACHE.clear()
        _CACHE[name] = workloads.make(name)
    return dict(_CACHE[name])


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.load()
    yield
    _CACHE.clear()


@pytest.mark.parametrize("name", ["identity", "headline", "headline_sharp", "top_p", "ties"])
def test_full_size_sampled_rows(name):
    w = _workload(name)
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
    binds = oracle.binding_filters(oracle.support(keys, w["top_k"][sample], w["top_p"][sample], w["min_p"][sample]), V)
    say(f"  logprob err {err:.2e}  side err {e_s:.2e}/{e_f:.2e}  dH rows rel {rh:.2e}  "
        f"|sum_v dW| {colsum:.2e} (max|dW| {scale:.2e})  -inf rows {int(np.isinf(lpa).sum())}; "
        f"binding filter on the sampled rows {binds}")
    assert err < LOGPROB_ATOL and e_s < 1e-4 and e_f < 5e-4 and rh < GRAD_RTOL
    # each term of a column sum is below max|dW|; fp32 dW rounding over V rows bounds the sum
    assert colsum < 1e-3 * scale * np.sqrt(V)
    assert np.isfinite(lpa[~np.isinf(lpa)]).all()


# ---------------------------------------------------------------- one full chunk, every element of dW
_SHARED = {}


def _oracle_rows(bounds):
    """Oracle forward and dlogits of rows [r0, r1) of the shared inputs
    (runs in a forked worker; BLAS limited to two threads there)."""
    from threadpoolctl import threadpool_limits
    r0, r1 = bounds
    S = _SHARED
    with threadpool_limits(2):
        rows = np.arange(r0, r1)
        f = oracle.forward(S["h"], S["W"], S["y"], S["temp"], S["k"], S["p"], S["mp"], keys=S["keys"][r0:r1],
                           rows=rows)
        dz = oracle.dlogits(S["h"], S["W"], S["y"], f, S["g"], S["temp"])
    nz = np.nonzero(dz)
    return (r0, f["n"], f["key_thr"], f["id_thr"], f["logprob"], f["near"], nz[0] + r0, nz[1], dz[nz])


def test_full_chunk_grad_weight_every_element():
    """grad_weight of one whole chunk (4,096 headline rows, full H and V)
    against the oracle element by element (relative Frobenius error), with a
    random upstream gradient per row, so a per-row or per-column scale error,
    a transposed or permuted operand, or a lost row shows.  The oracle runs on
    the GPU's keys of every row (support bit for bit first) in 8 forked
    workers; dz has at most 20 nonzeros per row here, so the two products
    dz^T h and dz W take it as a sparse matrix (the same sums)."""
    import scipy.sparse as sp
    w = _workload("headline")
    T, H, V = 4096, w["H"], w["V"]
    for key in ("h", "temperature", "top_k", "top_p", "min_p"):
        w[key] = np.ascontiguousarray(w[key][:T])
    say(f"full chunk dW: T={T} H={H} V={V}")
    G0 = to_gpu(w, np.zeros(T, np.int64))
    keys_d = binding.scaled_logits(G0["h"], G0["W"], G0["temperature"])
    # targets: the top token (every 7th row the 4th, every 10th row a uniform id, mostly out of support)
    top = torch.topk(keys_d, 4, dim=1).indices.cpu().numpy()
    y = np.where(np.arange(T) % 7 == 3, top[:, 3], top[:, 0])
    y = np.where(np.arange(T) % 10 == 0, w["target_uniform"][:T], y)
    keys = keys_d.cpu().numpy()
    del keys_d
    G = to_gpu(w, y)
    del G0
    g = np.random.Generator(np.random.PCG64(77)).standard_normal(T).astype(np.float32)
    lp, st = binding.forward(G["h"], G["W"], G["target"], **meta_of(G))
    gh, gw = binding.backward(G["h"], G["W"], G["target"], st, torch.from_numpy(g).to(dev()), **meta_of(G))
    torch.cuda.synchronize()
    info = binding.decode_state(st)
    gwc = gw.cpu().numpy()
    ghc = gh.float().cpu().numpy()
    lpg = lp.cpu().numpy()
    del gw, gh, G
    torch.cuda.empty_cache()
    W64 = w["W"].astype(np.float64)
    _SHARED.update(h=w["h"], W=W64, y=y, temp=w["temperature"], k=w["top_k"], p=w["top_p"], mp=w["min_p"],
                   keys=keys, g=g.astype(np.float64))
    nproc = 8
    bounds = [(i * T // nproc, (i + 1) * T // nproc) for i in range(nproc)]
    try:
        with multiprocessing.get_context("fork").Pool(nproc) as pool:
            parts = pool.map(_oracle_rows, bounds)
    finally:
        _SHARED.clear()
    n = np.concatenate([q[1] for q in parts])
    kt = np.concatenate([q[2] for q in parts])
    it = np.concatenate([q[3] for q in parts])
    lpo = np.concatenate([q[4] for q in parts])
    near = np.concatenate([q[5] for q in parts])
    assert not near.any()
    assert np.array_equal(info["n"], n) and np.array_equal(info["key_thr"], kt) and np.array_equal(info["id_thr"], it)
    fin = np.isfinite(lpo)
    assert np.array_equal(np.isfinite(lpg), fin)
    err = float(np.abs(lpg[fin] - lpo[fin]).max())
    dz = sp.csr_matrix((np.concatenate([q[8] for q in parts]),
                        (np.concatenate([q[6] for q in parts]), np.concatenate([q[7] for q in parts]))),
                       shape=(T, V))
    dH, dW = oracle.gradient_products(dz, w["h"], W64)
    rw = rel_fro(gwc, dW)
    rh = rel_fro(ghc, dH)
    say(f"  support equal on {T} rows ({int((~fin).sum())} out of support), logprob err {err:.2e}, "
        f"dz nonzeros {dz.nnz}, dW rel {rw:.2e}, dH rel {rh:.2e}")
    assert err < LOGPROB_ATOL and rw < GRAD_RTOL and rh < GRAD_RTOL
    # the rows of dW no support reaches are exactly zero on the GPU too
    untouched = np.ones(V, bool)
    untouched[np.unique(dz.indices)] = False
    assert not gwc[untouched].any()
