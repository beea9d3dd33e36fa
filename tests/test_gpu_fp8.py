"""GPU parity of the fp8 lane: an e4m3 LM head with per-row weight scales,
the hidden rows quantized per row by the library.

  * the quantizer's codes and scales bit for bit against the oracle, on
    random rows and on rows that land on every rounding tie;
  * the projection bit for bit on operands whose products and sums are exact
    in fp32 (the matrix cores' operand layout, the scales and the tails);
  * keys within fp32 accumulation error of the oracle's fp64 logits;
  * the workloads' support (bit for bit on the GPU's own keys), logprob and
    gradients, as for the bf16 lane; the backward's recomputed keys equal the
    forward's bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import (GRAD_RTOL, check_logprob, check_recomputed_keys, check_support, check_support_lists,
                         check_tile_lists, dev,
                         meta_of, rel_fro, say, targets, to_gpu)
from sampling_transform_logprob_amd import binding, workloads
from sampling_transform_logprob_amd.workloads import round_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.load()


def _bf16(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(dev()).to(torch.bfloat16)


def _tie_row(H):
    """A row whose maximum is 448 (scale exactly 1), then values halfway
    between neighbouring e4m3 values in several binades, signed."""
    ties = [1.0625, 1.1875, 17.0, 19.0, 2.0 ** -10, 3 * 2.0 ** -10, 15 * 2.0 ** -10, 248.0, 432.0, 0.5 + 1 / 32,
            2.0 ** -7 + 2.0 ** -10]
    r = np.zeros(H, np.float32)
    r[0] = 448.0
    r[1:1 + len(ties)] = ties
    r[1 + len(ties):1 + 2 * len(ties)] = [-t for t in ties]
    return r


@pytest.mark.parametrize("R,H", [(37, 16), (300, 5120), (5, 2064)])
def test_quantize_rows_bitwise(R, H):
    rng = np.random.Generator(np.random.PCG64(R * 7 + H))
    x = round_bf16(rng.standard_normal((R, H)).astype(np.float32) * rng.uniform(1e-3, 1e3, (R, 1)).astype(np.float32))
    x[0] = 0.0                                            # an all-zero row: scale 1, every code 0
    x[1] = _tie_row(H) if H >= 32 else x[1]
    if R > 3:
        x[2] = round_bf16(np.float32(2.0 ** -100) * rng.standard_normal(H).astype(np.float32))  # tiny values
        x[3, :] = -3.0                                     # constant row: every code the largest
    say(f"fp8 quantize: R={R} H={H}")
    codes, scales = binding.fp8_quantize_rows(_bf16(x))
    rc, ra = oracle.fp8_quantize_rows(x)
    assert np.array_equal(scales.cpu().numpy().view(np.uint32), ra.view(np.uint32))
    c = codes.cpu().numpy()
    bad = np.argwhere(c != rc)
    assert bad.size == 0, f"codes differ at {bad[:5].tolist()}: gpu {c[tuple(bad[0])]:#x} oracle {rc[tuple(bad[0])]:#x}"
    if H >= 32:
        assert c[1, 0] == 0x7E                            # 448
        assert list(c[1, 1:12]) == [0x38, 0x3A, 0x58, 0x5A, 0x00, 0x02, 0x08, 0x78, 0x7E, 0x30, 0x04]


def _exact_operands(T, H, V, seed):
    """Hidden rows of multiples of 1/16 up to 7 (each row's maximum is 7, so
    its scale is 7/448 = 2^-6 and its codes are the values times 64) and
    weight codes of values (1 + m/8) 2^e, e in [-1, 2], with power-of-two row
    scales: every product and every partial sum is exact in fp32 (the sums
    stay below 2^21 in steps of 1/4)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    vals = sorted({(8 + m) / 8 * 2.0 ** e for m in range(8) for e in range(-1, 3) if (8 + m) / 8 * 2.0 ** e <= 7})
    pool = np.array([0.0] + vals + [-v for v in vals], np.float32)
    h = rng.choice(pool, (T, H)).astype(np.float32)
    h[np.arange(T), rng.integers(0, H, T)] = np.float32(7.0) * rng.choice(np.float32([-1, 1]), T)
    e = rng.integers(6, 10, (V, H)).astype(np.uint8)
    m = rng.integers(0, 8, (V, H)).astype(np.uint8)
    s = rng.integers(0, 2, (V, H)).astype(np.uint8)
    W8 = (s << 7) | (e << 3) | m
    W8[rng.random((V, H)) < 0.05] = 0
    w_scale = np.exp2(rng.integers(-8, -5, V)).astype(np.float32)
    return h, W8, w_scale


@pytest.mark.parametrize("T,H,V", [(300, 384, 700), (64, 128, 256), (17, 16, 37)])
def test_exact_operand_projection_is_bitwise(T, H, V):
    """Three and one k-tiles of 128 (an odd count pads with a zero tile), a
    single 16-wide k-chunk, ragged vocabulary and token tiles."""
    h, W8, sw = _exact_operands(T, H, V, T + H + V)
    z64 = oracle.fp8_logits(h, W8, sw)
    assert np.array_equal(z64.astype(np.float32).astype(np.float64), z64)    # exact in fp32 by construction
    say(f"fp8 exact operands: T={T} H={H} V={V}")
    keys = binding.scaled_logits(_bf16(h), torch.from_numpy(W8).to(dev()), None,
                                 weight_scale=torch.from_numpy(sw).to(dev())).cpu().numpy()
    bad = np.argwhere(keys != z64.astype(np.float32))
    assert bad.size == 0, f"{bad.shape[0]} keys differ, first at {bad[:4].tolist()}"


def test_projection_accuracy():
    w = workloads.make("headline_fp8", T=96)
    V = 8192
    W8, sw = w["W"][:V], w["w_scale"][:V]
    say(f"fp8 projection accuracy: T=96 H={w['H']} V={V}")
    keys = binding.scaled_logits(_bf16(w["h"]), torch.from_numpy(W8).to(dev()),
                                 torch.from_numpy(w["temperature"]).to(dev()),
                                 weight_scale=torch.from_numpy(sw).to(dev())).cpu().numpy()
    t = w["temperature"].astype(np.float64)[:, None]
    z64 = oracle.fp8_logits(w["h"], W8, sw)
    h8, a = oracle.fp8_quantize_rows(w["h"])
    scale = (np.abs(oracle.e4m3_decode(h8)) @ np.abs(oracle.e4m3_decode(W8)).T) * sw[None, :] * a[:, None] / t
    err = (np.abs(keys - z64 / t) / scale).max()
    say(f"  max error relative to sum |products|: {err:.2e}")
    assert err < 1e-5


def _fp8_case(name, T, V, dense=False):
    w = workloads.make(name, T=T)
    if V < w["V"]:
        w["W"], w["w_scale"], w["V"] = w["W"][:V], w["w_scale"][:V], V
        w["target_uniform"] = w["target_uniform"] % V
    if dense:                                    # top-p alone: supports of thousands, the dense row class
        w["top_k"][:] = 0
        w["top_p"][:] = 0.95
    return w


@pytest.mark.parametrize("name,T,V,dense", [("tiny_fp8", 64, 1000, False), ("headline_fp8", 300, 30000, False),
                                            ("headline_fp8", 200, 20000, True)])
def test_fp8_workload_parity(name, T, V, dense):
    w = _fp8_case(name, T, V, dense)
    say(f"fp8 parity {name}: T={T} H={w['H']} V={V} dense={dense}")
    y = targets(w)
    G = to_gpu(w, y)
    ws = G["weight_scale"]
    lp, st = binding.forward(G["h"], G["W"], G["target"], **meta_of(G), weight_scale=ws, chunk_rows=128)
    g = np.full(T, -1.0 / T)
    gg = torch.from_numpy(g.astype(np.float32)).to(dev())
    gh, gw = binding.backward(G["h"], G["W"], G["target"], st, gg, **meta_of(G), weight_scale=ws,
                              vocab_slice=7168 if V > 7168 else 0)
    keys = binding.scaled_logits(G["h"], G["W"], G["temperature"], weight_scale=ws)
    rk = binding.recompute_keys(G["h"], G["W"], G["target"], st, gg, **meta_of(G), weight_scale=ws)
    torch.cuda.synchronize()
    kc = keys.cpu().numpy()
    info = binding.decode_state(st)
    check_tile_lists(info, kc, V)
    check_support_lists(info, kc)
    check_recomputed_keys(rk.cpu().numpy(), kc, info, g, y, V, "fp8")
    ref = oracle.forward(w["h"], w["W"], y, w["temperature"], w["top_k"], w["top_p"], w["min_p"], keys=kc,
                         lane="fp8", w_scale=w["w_scale"])
    near = check_support(info, ref, name)
    err = check_logprob(lp.cpu().numpy(), ref)
    dH, dW = oracle.backward(w["h"], w["W"], y, ref, g, w["temperature"], w_scale=w["w_scale"])
    assert gh.dtype == torch.bfloat16
    rh, rw = rel_fro(gh.float().cpu().numpy(), dH), rel_fro(gw.cpu().numpy(), dW)
    say(f"  near={near} logprob err={err:.2e} dH rel={rh:.2e} dW rel={rw:.2e} "
        f"supports: min {info['n'].min()} max {info['n'].max()}")
    assert near == 0
    if dense:
        assert (info["n"] > 128).sum() > T // 2          # the dense class is exercised
    assert rh < GRAD_RTOL and rw < GRAD_RTOL
    # chunking does not change a bit (the re-projection gathers codes)
    lp2, st2 = binding.forward(G["h"], G["W"], G["target"], **meta_of(G), weight_scale=ws, chunk_rows=0)
    assert torch.equal(lp2.view(torch.int32), lp.view(torch.int32)) and torch.equal(st2, st)


def test_fp8_rows_the_candidates_cannot_decide_are_reprojected():
    """Half the rows put their 4 largest logits on tokens 0..3 (one lane of
    tile 0), so the candidates cannot decide them: their hidden codes are
    gathered and projected again with their row scales."""
    T, H, V = 300, 256, 40000
    rng = np.random.Generator(np.random.PCG64(23))
    W = (rng.standard_normal((V, H)) * 0.02).astype(np.float32)
    u = rng.standard_normal(H).astype(np.float32)
    u /= np.linalg.norm(u)
    W[:4] = u[None, :] * np.float32([0.9, 0.85, 0.8, 0.75])[:, None]
    # the weight's codes and row scales through torch's own e4m3 conversion
    sw = (np.abs(W).max(1) / 448.0).astype(np.float32)
    W8 = torch.from_numpy(W / sw[:, None]).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    h = rng.standard_normal((T, H)).astype(np.float32)
    crowd = np.arange(T) % 2 == 0
    h[crowd] += (8.0 * u)[None, :]
    h = round_bf16(h)
    w = dict(h=h, W=W8, w_scale=sw, temperature=np.full(T, 0.7, np.float32), top_k=np.full(T, 20, np.int32),
             top_p=np.full(T, 0.9, np.float32), min_p=np.zeros(T, np.float32), dtype="fp8",
             u=np.random.Generator(np.random.PCG64(4)).random(T), filtered=True, V=V)
    y = targets(w)
    G = to_gpu(w, y)
    ws = G["weight_scale"]
    say(f"fp8 candidates with re-projection: T={T} V={V}")
    lp, st = binding.forward(G["h"], G["W"], G["target"], **meta_of(G), weight_scale=ws, chunk_rows=128)
    keys = binding.scaled_logits(G["h"], G["W"], G["temperature"], weight_scale=ws)
    torch.cuda.synchronize()
    kc = keys.cpu().numpy()
    ref = oracle.forward(h, W8, y, w["temperature"], w["top_k"], w["top_p"], w["min_p"], keys=kc, lane="fp8",
                         w_scale=sw)
    assert check_support(binding.decode_state(st), ref, "fp8 crowded") == 0
    check_logprob(lp.cpu().numpy(), ref)
    assert (kc[crowd].argsort(1)[:, -4:] < 4).all()
    lp1, st1 = binding.forward(G["h"][:40], G["W"], G["target"][:40],
                               **{k: v[:40] for k, v in meta_of(G).items()}, weight_scale=ws, chunk_rows=1)
    assert torch.equal(lp1.view(torch.int32), lp[:40].view(torch.int32)) and torch.equal(st1, binding.state_prefix(st, 40))
