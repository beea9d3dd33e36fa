"""Bit-exact support of the GPU selection kernel on adversarial fp32 key rows.

``stce_support_from_logits`` runs the forward's selection kernel on given
keys; the oracle computes the support of the very same keys.  The rows cover
every path of the kernel: whole-row windows (V <= CAP), bounded candidates
(top-k from tile maxima, min-p), the value histogram, and the radix
refinement used when a histogram bin holds more tokens than the window
(long tie groups, very peaked rows), plus the identities of the program."""
import math

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import dev, say
from sampling_transform_logprob_amd import binding

pytestmark = pytest.mark.gpu

CAP = 3712   # the selection kernel's window capacity (tokens gathered into LDS)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.load()


def _check(keys, k, p, mp, y=None, label=""):
    keys = np.ascontiguousarray(keys, np.float32)
    R, V = keys.shape
    k = np.asarray(k, np.int32)
    p = np.asarray(p, np.float32)
    mp = np.asarray(mp, np.float32)
    y = np.zeros(R, np.int64) if y is None else np.asarray(y, np.int64)
    say(f"support {label}: R={R} V={V}")
    lp, st = binding.support_from_logits(torch.from_numpy(keys).to(dev()), torch.from_numpy(y).to(dev()),
                                         torch.from_numpy(k).to(dev()), torch.from_numpy(p).to(dev()),
                                         torch.from_numpy(mp).to(dev()))
    info = binding.decode_state(st)
    lpc = lp.cpu().numpy()
    ref = oracle.support(keys, k, p, mp)
    ok = ~ref["near"]
    assert ref["near"].sum() == 0, f"{label}: {ref['near'].sum()} rows within rounding"
    bad = np.nonzero(info["n"] != ref["n"])[0]
    assert bad.size == 0, f"{label}: n differs at rows {bad[:8]}: gpu {info['n'][bad[:8]]} oracle {ref['n'][bad[:8]]}"
    filt = (info["flags"] & binding.FLAG_FILTERED) != 0
    bad = np.nonzero(filt & ((info["key_thr"] != ref["key_thr"]) | (info["id_thr"] != ref["id_thr"])))[0]
    assert bad.size == 0, f"{label}: boundary differs at rows {bad[:8]}"
    # selected logprob on the support, from the same keys
    for r in range(R):
        mask = oracle.in_support(keys[r], int(ref["key_thr"][r]), int(ref["id_thr"][r])) if filt[r] else \
            np.ones(V, bool)
        s64 = keys[r].astype(np.float64)
        mx = s64[mask].max()
        lse = mx + math.log(np.exp(s64[mask] - mx).sum())
        want = min(s64[y[r]] - lse, 0.0) if mask[y[r]] else -math.inf
        if math.isinf(want):
            assert lpc[r] == -np.inf, (label, r)
        else:
            assert abs(lpc[r] - want) < 1e-4, (label, r, lpc[r], want)
    return info


def _grid(rng, V, R, ties):
    keys = (rng.standard_normal((R, V)) * rng.uniform(0.3, 4, (R, 1))).astype(np.float32)
    if ties:
        keys = (np.round(keys * 4) / 4).astype(np.float32)
    return keys


@pytest.mark.parametrize("V", [4, 8, 300, 1000, CAP, CAP + 4, 4096, 5000, 40000])
def test_random_rows_all_filter_mixes(V):
    rng = np.random.Generator(np.random.PCG64(V))
    R = 96
    keys = _grid(rng, V, R, ties=(V % 2 == 0))
    ks = np.array([0, 1, 2, 20, 64, V - 1, V, V + 5, CAP - 1, CAP + 1, 4097])
    ps = np.array([1.0, 0.9, 0.5, 1e-6, np.nextafter(np.float32(1), np.float32(0)), 0.99])
    mps = np.array([0.0, 0.0, 0.1, 1.0, 1e-3])
    k = np.maximum(ks[rng.integers(0, len(ks), R)], 0)
    p = ps[rng.integers(0, len(ps), R)]
    mp = mps[rng.integers(0, len(mps), R)]
    y = rng.integers(0, V, R)
    _check(keys, k, p, mp, y, f"random V={V}")


def test_identities():
    rng = np.random.Generator(np.random.PCG64(3))
    V = 7000
    keys = _grid(rng, V, 8, ties=True)
    info = _check(keys, [0, V, V + 3, 0, 0, 0, 0, 0], [1.0] * 8, [0.0] * 8, label="identity rows")
    assert np.all(info["n"] == V)


def test_top_p_one_despite_fp32_overshoot():
    V = 6000
    keys = np.zeros((2, V), np.float32)      # equal keys: fp32 running sums of 1/V drift past 1
    info = _check(keys, [0, 0], [1.0, 1.0], [0.0, 0.0], label="overshoot")
    assert np.all(info["n"] == V)


def test_tie_groups_longer_than_the_window():
    V = 20000
    keys = np.zeros((6, V), np.float32)
    keys[1, :] = 1.5
    keys[2, ::2] = 2.0                         # two long tie groups
    keys[3, 5000:15000] = 3.0
    keys[4] = np.where(np.arange(V) % 3 == 0, -0.0, 0.0)   # signed zeros are one key
    keys[5, 17] = 5.0
    k = [10000, 1, 9999, 7000, 4500, 12000]
    _check(keys, k, [1.0, 1.0, 1.0, 0.3, 1.0, 1.0], [0.0] * 6, np.arange(6) * 997, "long ties")


def test_peaked_rows_need_radix_refinement():
    rng = np.random.Generator(np.random.PCG64(5))
    V = 60000
    keys = (rng.random((4, V)) * 1e-3).astype(np.float32)   # a narrow cluster...
    keys[:, 123] = 40.0                                      # ...and one far outlier
    k = [30000, 0, 25000, 0]
    p = [1.0, 1.0, 0.9, 1.0]
    mp = [0.0, 1e-30, 0.0, 0.0]
    keys[3, :] = np.float32(7.0)
    keys[3, ::7] = np.nextafter(np.float32(7.0), np.float32(8.0))
    _check(keys, k, p, mp, [123, 5, 77, 14], "peaked")


def test_min_p_keeps_whole_tie_groups_and_uses_unfiltered_max():
    V = 9000
    keys = np.full((3, V), -5.0, np.float32)
    keys[:, :100] = 0.0
    keys[:, 100:2000] = np.float32(math.log(0.1))           # exactly at the min-p threshold in fp32
    keys[1, 7] = 3.0
    info = _check(keys, [0, 0, 50], [1.0, 1.0, 1.0], [0.1, 0.1, 0.1], label="min-p groups")
    assert info["n"][0] in (100, 2000)


def test_top_p_near_the_top_k_mass_takes_the_exact_path():
    """Rows whose top-k mass lies within 1e-3 of p of the row mass cannot be
    certified from the fp32 partials; the kernel must then take the exact
    fp64 full-row mass, on both sides of the crossing."""
    rng = np.random.Generator(np.random.PCG64(17))
    V, R = 20000, 24
    keys = rng.standard_normal((R, V)).astype(np.float32)
    keys[:, :2] = 10.0
    s64 = keys.astype(np.float64)
    frac = np.exp(s64[:, :2] - 10.0).sum(1) / np.exp(s64 - 10.0).sum(1)   # mass of the top two
    rel = np.tile([-3e-4, -1e-5, -1e-7, 1e-7, 1e-5, 3e-4, -5e-3, 5e-3], R // 8)
    p = (frac * (1 + rel)).astype(np.float32)
    info = _check(keys, np.full(R, 2), p, np.zeros(R), np.zeros(R, np.int64), "top-p band")
    # p slightly below the top-two mass: top-p crosses at the second token (a
    # tie with the first: n = 2 either way); p above it: top-k 2 binds
    assert np.all(info["n"] <= 2)


def test_k_bounded_rows_read_only_candidate_tiles():
    """Top-k rows whose candidates sit in a few tiles, next to rows whose
    tile list overflows (min-p keeping most of the row)."""
    rng = np.random.Generator(np.random.PCG64(23))
    V, R = 150000, 16
    keys = (rng.standard_normal((R, V)) * 0.01).astype(np.float32)
    hot = rng.integers(0, V, (R, 30))
    for r in range(R):
        keys[r, hot[r]] = rng.uniform(5, 6, 30).astype(np.float32)
    k = np.array([20, 1, 30, 31] * 4)
    p = np.array([1.0, 0.8, 0.999, 1.0] * 4, np.float32)
    mp = np.array([0.0, 0.0, 0.0, 1e-9] * 4, np.float32)
    _check(keys, k, p, mp, hot[:, 0], "candidate tiles")


def test_vocabularies_beyond_the_tile_bound_search():
    """V > 2 * CAP * 256: more tile maxima than the bitwise k-th-largest search
    handles (its list lives in the window's LDS), so top-k rows fall back to
    the value histogram (and radix refinement on ties).  Also a vocabulary
    just below that limit, where the search still runs."""
    rng = np.random.Generator(np.random.PCG64(29))
    for V, R in ((2 * CAP * 256 + 256, 6), (2 * CAP * 256 - 256, 6)):
        keys = (rng.standard_normal((R, V)) * rng.uniform(0.5, 3, (R, 1))).astype(np.float32)
        keys[1] = np.round(keys[1] * 2) / 2                     # heavy ties
        k = np.array([20, 1000, 64, 0, 5, 3000], np.int32)
        p = np.array([1.0, 0.9, 1.0, 0.5, 0.99, 1.0], np.float32)
        mp = np.array([0.0, 0.0, 0.05, 0.0, 0.0, 1e-4], np.float32)
        y = np.array([int(np.argmax(keys[r])) for r in range(R)])
        _check(keys, k, p, mp, y, f"V={V}")


def test_min_p_tiles_above_index_65535():
    """V = 2^24 + 1024 has 65,540 vocabulary tiles.  A min-p row whose
    passing tokens sit only in tiles 65,536 .. 65,539 takes the candidate-tile
    list; the list must keep those indices whole (a 16-bit index would wrap
    them to tiles 0 .. 3 and read the wrong keys).  A top-k row at this V
    takes the value histogram (too many tile maxima for the bound search)."""
    V = (1 << 24) + 1024
    rng = np.random.Generator(np.random.PCG64(41))
    keys = rng.uniform(-10.0, -9.0, (3, V)).astype(np.float32)
    hi = 1 << 24                                    # first token of tile 65,536
    for r in range(3):
        keys[r, hi + 10] = 5.0                      # tile 65,536: the row maximum
        keys[r, hi + 300] = 4.8                     # tile 65,537
        keys[r, hi + 900] = 4.5                     # tile 65,539
        keys[r, 77] = 4.0                           # tile 0: below the min-p bar of rows 0 and 1
    k = np.array([0, 0, 2], np.int32)
    p = np.array([1.0, 0.9, 1.0], np.float32)
    mp = np.array([0.5, 0.5, 0.0], np.float32)      # ln 0.5 = -0.69: keys >= 4.31 pass
    y = np.array([hi + 900, hi + 10, hi + 300])
    info = _check(keys, k, p, mp, y, "tiles above 65535")
    assert info["n"][0] == 3 and info["id_thr"][0] == hi + 900
    assert info["n"][2] == 2 and info["id_thr"][2] == hi + 300
