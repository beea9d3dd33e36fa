"""Seeded synthetic workloads for the scoring core (inputs only).

This module draws random inputs and nothing else: it holds none of the
scoring arithmetic, so the fp64 oracle and the HIP library can both be fed
from it.  Every array comes from ``numpy.random.Generator(PCG64)`` children
of one seed, so a smaller ``T`` gives a prefix of the rows of the full size
(the weight matrix does not depend on ``T``).

Shapes follow the workloads of the pages: an untied LM head of a 151,936-token
vocabulary, 16,384-token micro-batches (align "architecture v2: proposal",
sections 5.1 and 5.4 A), and rollouts sampled with per-row temperature and
top-k / top-p / min-p (xorl pull request 74).

Operands are returned as float32 numpy arrays whose values are exactly
representable in the named dtype (bf16 values are rounded to nearest-even).
The fp8 configurations instead return the weight as e4m3 codes (uint8) with
one fp32 scale per vocabulary row, drawn directly as bit fields (see
``_e4m3_codes``), and bf16 hidden states.
Targets are not drawn here for the filtered configurations: drawing one from
a row's filtered distribution needs the scoring arithmetic, so the caller
turns the uniforms ``u`` into targets (the tests through the oracle).
"""
from __future__ import annotations

import numpy as np

# name -> shape, dtype, seed, per-row program
CONFIGS = {
    # fp32 operands; every filter mixed per row
    "tiny": dict(T=64, H=128, V=1000, dtype="f32", seed=1),
    # plain cross-entropy: temperature 1, no filter, uniform targets
    "identity": dict(T=4096, H=2048, V=32000, dtype="bf16", seed=2),
    # full-row top-p with per-row temperature
    "top_p": dict(T=8192, H=4096, V=128256, dtype="bf16", seed=3),
    # the headline shape: temperature 0.7, top-k 20, top-p 0.8
    "headline": dict(T=16384, H=5120, V=151936, dtype="bf16", seed=4),
    # the headline program on a sharper head (W std x3): logits/T std about 6,
    # so top-p 0.8 binds inside top-k 20 on most rows (a parity variant)
    "headline_sharp": dict(T=16384, H=5120, V=151936, dtype="bf16", seed=6, w_std=0.06),
    # 4-bit weight levels with duplicated rows: many bitwise-equal logits
    "ties": dict(T=32768, H=7168, V=129280, dtype="bf16", seed=5),
    # the headline shape and program on an e4m3 head with per-row scales
    "headline_fp8": dict(T=16384, H=5120, V=151936, dtype="fp8", seed=7),
    # small e4m3 head, every filter mixed per row (the program of "tiny")
    "tiny_fp8": dict(T=64, H=128, V=1000, dtype="fp8", seed=8),
}

# scale of the fp8 weight rows: the drawn codes have an rms of about 142, so
# 1.4e-4 gives dequantized weights of rms about 0.02 (the bf16 headline's)
FP8_W_SCALE = 1.4e-4


def _e4m3_codes(rng, shape) -> np.ndarray:
    """e4m3 codes drawn as bit fields from one uniform 16-bit word each:
    bits 0-2 the mantissa field, bit 3 the sign, bits 4-15 give
    tz = the count of trailing zero bits (0 .. 12, geometric: P(tz = k) =
    2^-(k+1)), and the exponent field is 14 - tz (values 2^(7 - tz) .. 1.875
    2^(7 - tz)), or 0 when tz = 12 (zero and subnormal codes).  Exponent
    field 15 is never drawn, so neither the codes above 240 nor the NaN codes
    occur."""
    w = rng.integers(0, 1 << 16, size=shape, dtype=np.uint16)
    top = (w >> np.uint16(4)).astype(np.uint16)
    tz_table = np.array([12] + [((k & -k).bit_length() - 1) for k in range(1, 4096)], np.uint8)
    tz = tz_table[top]
    e = np.where(tz == 12, 0, 14 - tz.astype(np.int16)).astype(np.uint8)
    return (((w >> np.uint16(3)) & np.uint16(1)).astype(np.uint8) << np.uint8(7)) | (e << np.uint8(3)) | (
        w & np.uint16(7)).astype(np.uint8)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even), as float32."""
    x = np.array(x, dtype=np.float32, copy=True)
    b = x.view(np.uint32)              # finite values: the sum cannot wrap
    b += np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))
    b &= np.uint32(0xFFFF0000)
    return x


def _children(seed: int, n: int = 6):
    return [np.random.Generator(np.random.PCG64(s)) for s in np.random.SeedSequence(seed).spawn(n)]


def make(name: str, T: int | None = None, seed: int | None = None) -> dict:
    """Inputs of configuration ``name`` with ``T`` rows (default: its full T).

    Returns a dict with ``h`` [T, H], ``W`` [V, H] (float32 arrays holding
    values of ``dtype``; for the fp8 configurations ``W`` holds e4m3 codes,
    uint8, ``w_scale`` [V] fp32 their row scales and ``h`` bf16 values),
    per-row ``temperature`` (fp32), ``top_k`` (int32,
    0 = off), ``top_p`` (fp32, 1 = off), ``min_p`` (fp32, 0 = off), ``u``
    (uniforms in [0, 1) for drawing targets), ``target_uniform`` (int64
    uniform ids), ``filtered`` (whether targets should come from the
    filtered distribution) and the shape fields.
    """
    cfg = dict(CONFIGS[name])
    T = int(cfg["T"] if T is None else T)
    H, V = cfg["H"], cfg["V"]
    rw, rh, rm, ru, rt, rp = _children(cfg["seed"] if seed is None else seed)
    bf16 = cfg["dtype"] in ("bf16", "fp8")
    w_scale = None

    if cfg["dtype"] == "fp8":
        W = _e4m3_codes(rw, (V, H))
        # per-row scales: FP8_W_SCALE times 2^U, U uniform in [-1/2, 1/2)
        w_scale = (FP8_W_SCALE * np.exp2(rp.random(V) - 0.5)).astype(np.float32)
    elif name == "ties":
        # 4-bit levels of N(0, 0.02^2) in steps of 2^-6, clamped to [-8, 7];
        # V rows drawn with replacement from V/6 distinct rows, so duplicated
        # rows give bitwise-equal logits (tie groups of random size).
        pool = rw.standard_normal((V // 6, H), dtype=np.float32) * np.float32(0.02)
        pool = np.clip(np.rint(pool * 64.0), -8, 7).astype(np.float32) / np.float32(64.0)
        W = pool[rp.integers(0, V // 6, size=V)]
    else:
        W = rw.standard_normal((V, H), dtype=np.float32) * np.float32(cfg.get("w_std", 0.02))
    h = rh.standard_normal((T, H), dtype=np.float32)
    if bf16:
        h = round_bf16(h)
        if w_scale is None:
            W = round_bf16(W)

    ones = np.ones(T, np.float32)
    if name in ("tiny", "tiny_fp8"):
        temp = rm.uniform(0.5, 1.5, T).astype(np.float32)
        top_k = np.where(rm.random(T) < 0.5, 0, 50).astype(np.int32)
        top_p = np.where(rm.random(T) < 0.5, 1.0, 0.9).astype(np.float32)
        min_p = np.where(rm.random(T) < 0.5, 0.0, 0.05).astype(np.float32)
    elif name == "identity":
        temp, top_k, top_p, min_p = ones, np.zeros(T, np.int32), ones.copy(), np.zeros(T, np.float32)
    elif name == "top_p":
        temp = rm.uniform(0.6, 1.2, T).astype(np.float32)
        top_k, top_p, min_p = np.zeros(T, np.int32), np.full(T, 0.95, np.float32), np.zeros(T, np.float32)
    elif name in ("headline", "headline_sharp", "headline_fp8"):
        temp = np.full(T, 0.7, np.float32)
        top_k, top_p, min_p = np.full(T, 20, np.int32), np.full(T, 0.8, np.float32), np.zeros(T, np.float32)
    elif name == "ties":
        temp = rm.uniform(0.3, 1.5, T).astype(np.float32)
        kind = rm.integers(0, 3, T)                  # 0 identity, 1 min-p, 2 top-k
        top_k = np.where(kind == 2, 64, 0).astype(np.int32)
        top_p = ones.copy()
        min_p = np.where(kind == 1, 0.1, 0.0).astype(np.float32)
    else:  # pragma: no cover
        raise KeyError(name)

    return dict(
        name=name, T=T, H=H, V=V, dtype=cfg["dtype"], h=h, W=W, w_scale=w_scale,
        temperature=temp, top_k=top_k, top_p=top_p, min_p=min_p,
        u=ru.random(T), target_uniform=rt.integers(0, V, size=T).astype(np.int64),
        filtered=name != "identity",
    )
