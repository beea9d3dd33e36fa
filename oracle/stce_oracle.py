"""Plain fp64 CPU oracle of the sampling-transform scoring core.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library (``sampling_transform_logprob_amd``) and imports nothing from it.

What it computes, and where each step comes from
------------------------------------------------
Sources are the text of the web pages this project was built from:

* [xorl#74] -- togethercomputer/xorl pull request 74, "Consolidate
  sampling-transform scoring on one shared chunked core; implement
  top-k/top-p/min-p replay for generic ce_modes".
* [align-v2] -- viai957/align, "align architecture v2: proposal",
  section 5.4 A ("Fused head + policy-gradient token loss").
* [nested-learning] -- nested-learning 0.2.0, ``nested_learning/training.py``,
  function ``compute_teach_signal`` (closed-form cross-entropy gradient).

The pipeline per scored row t (a token of a replayed rollout):

1. logits ``z = h W^T``                         ([xorl#74] "What this PR does" 2:
   chunked projection; [align-v2] 5.4 A: logits kept in fp32, not rounded
   to bf16).  Here: exact fp64 product of the (bf16 or fp32) operands.
2. temperature first: keys ``s = fl32(fl32(z) / T_t)``, per row, after the
   projection ([xorl#74] "What this PR does" 1, "temperature-first"; the
   self-review pass documents the per-row post-GEMM convention).  fp64 has
   53 >= 2*24+2 bits, so rounding the fp64 quotient of two fp32 numbers to
   fp32 gives the correctly rounded fp32 quotient.
3. the support program on the fp32 keys ([xorl#74] "What this PR does" 1):
   order by key descending with the lower token id first among equal keys
   (stable token-id tie-break); top-k keeps the first k; top-p keeps the
   shortest prefix whose mass reaches p of the full-row mass, the crossing
   token included; min-p keeps tokens whose probability is at least min_p
   times that of the row maximum taken BEFORE any filter; top_p == 1 is the
   identity and never looks at a running sum.  The three filters are read as
   one joint intersection on the single temperature-scaled, unfiltered
   distribution (each is a prefix of the same order; the support is the
   shortest of the three prefixes).  Decision arithmetic is fp64 on the fp32
   keys.
4. selected logprob on the filtered support, clamped to <= 0 (self-review
   pass of [xorl#74]); a target outside the support scores -inf and gets an
   exactly zero gradient ([xorl#74] "What this PR does" 4).
5. closed-form VJP ([xorl#74] "What this PR does" 2: recompute closed-form
   VJP; [nested-learning] ``compute_teach_signal``; [align-v2] 5.4 A sign
   convention): ``d logprob / d z_j = (1[j = y] - q_j) / T`` with ``q`` the
   softmax of ``z / T`` restricted to the support, then ``dH = dz W`` and
   ``dW = dz^T h``.

A policy-gradient token loss on top of the selected logprob ([align-v2]
5.4 A, "Why the in-chunk form works for this loss"): with the ratio
``r = exp(logprob - logprob_old)`` and advantage ``A``, the loss sign (the
quantity an optimizer minimises) has ``d loss / d z = c (q - onehot) / T``,
i.e. ``d loss / d logprob = -c``, where
  CISPO:              c = A * sg(min(r, 1 + eps_high))   (no lower bound)
  clipped surrogate:  c = A * r * 1[the unclipped term is the minimum]
so the per-token losses are ``-A sg(min(r, 1+eps_high)) logprob`` and
``-min(r A, clip(r, 1-eps_low, 1+eps_high) A)``, each times a caller scale
(the reciprocal of a constant denominator).  The gradient then flows
through the same VJP as the logprob with ``g = d loss / d logprob``.

A second temperature convention ([xorl#74] self-review pass, which records
that a scalar temperature applied before the projection and a per-row one
applied after it are two documented conventions; "What this PR does" 1:
temperature is applied first, at the dtype boundary of the lane).  The pages
name it without its formula; read plainly: one scalar T divides the hidden
state before the projection, in fp32, and the quotient is rounded to the
operand dtype, ``h' = round(fl32(h) / T)``; the keys are then
``s = fl32(h' W^T)`` (no per-row division) and the VJP carries the 1/T to the
hidden state, ``dH = (dz W) / T`` with ``dz = g (onehot - q)``, and
``dW = dz^T h'`` (the rounding of ``h'`` passes gradients unchanged).
``pre_gemm_hidden`` and ``backward_pre_gemm`` below; ``forward`` takes ``h'``
with no per-row temperature.

A bf16 value lane ([xorl#74] deduplication and review passes: one model
family's exact head runs its value program in bf16 from end to end, with a
bf16 base projection, its own temperature dtype boundary and a bf16 selected
logprob, the expected logprob dtype being part of the family's contract).
The pages give no formula; read plainly, every value the program hands on
is a bf16 tensor: the projection's fp32 result is rounded to bf16,
``z_b = bf16(fl32(h W^T))``; the temperature divides that value in fp32 and
the quotient is rounded to bf16 again, ``s = bf16(fl32(z_b / T))``; the
support and the log-sum-exp are taken on these keys (accumulated at higher
precision, as a bf16 log-softmax does), and the selected logprob is rounded
to bf16 at the end.  The VJP is the one of ``s_y - lse_S(s)`` with the two
roundings passing gradients unchanged, so ``q`` comes from the bf16 keys.
``bf16_lane_keys`` and ``forward(lane="bf16")`` / ``backward(lane="bf16")``.

Values (logprob, gradients) use the unrounded fp64 logits ``u = z / T``.
Support decisions use only the fp32 keys, so a caller may pass the keys of
another implementation (``keys=``) to compare supports bit for bit.
"""
from __future__ import annotations

import math

import numpy as np

_SIGN = np.uint32(0x80000000)

# Relative margin under which a top-p or min-p decision is reported as
# "within rounding" (several answers are then defensible).
MARGIN = 1e-12


# --------------------------------------------------------------------------
# keys
# --------------------------------------------------------------------------
def canonical_f32(s32: np.ndarray) -> np.ndarray:
    """fp32 copy with -0.0 replaced by +0.0 (the two compare equal)."""
    s = np.array(s32, dtype=np.float32, copy=True)
    s[s == 0] = np.float32(0.0)
    return s


def order_keys(s32: np.ndarray) -> np.ndarray:
    """Order-preserving uint32 image of finite fp32 values (-0 -> +0).

    A larger float maps to a larger unsigned key: negative floats have their
    bits inverted, non-negative floats get the sign bit set.
    """
    s = canonical_f32(s32)
    assert np.all(np.isfinite(s)), "oracle inputs must be finite"
    b = s.view(np.uint32)
    return np.where(b & _SIGN, ~b, b | _SIGN).astype(np.uint32)


def scale_logits(z: np.ndarray, temperature: np.ndarray) -> np.ndarray:
    """Keys ``fl32(fl32(z) / T)`` per row (temperature first, post-projection)."""
    z32 = np.asarray(z, dtype=np.float64).astype(np.float32)
    t = np.asarray(temperature, dtype=np.float32).astype(np.float64)
    q = z32.astype(np.float64) / t[:, None]
    return canonical_f32(q.astype(np.float32))


def chunk_logits(h: np.ndarray, W: np.ndarray) -> np.ndarray:
    """``z = h W^T`` in fp64 (the operands are widened exactly)."""
    return np.asarray(h, dtype=np.float64) @ np.asarray(W, dtype=np.float64).T


# --------------------------------------------------------------------------
# support program (one row)
# --------------------------------------------------------------------------
def order_row(s_row: np.ndarray) -> np.ndarray:
    """Permutation pi: key descending, lower token id first among equal keys."""
    s = canonical_f32(s_row).astype(np.float64)
    ids = np.arange(s.shape[0])
    return np.lexsort((ids, -s))


def support_row(s_row: np.ndarray, top_k: int, top_p: float, min_p: float) -> dict:
    """Support of one row of fp32 keys.

    Returns a dict with the support size ``n``, the boundary token (the last
    token of the support in order pi) as ``id_thr`` with its key ``key_thr``,
    the per-filter prefix lengths, the fp64 decision masses and a flag
    ``near`` set when a binding top-p / min-p decision lies within ``MARGIN``
    (relative) of flipping.
    """
    s = canonical_f32(s_row)
    V = s.shape[0]
    s64 = s.astype(np.float64)
    pi = order_row(s)
    m = s64[pi[0]]                       # row maximum before any filter
    w = np.exp(s64[pi] - m)              # decision masses, in order pi
    cum = np.cumsum(w)
    Z = cum[-1]
    k = int(top_k)
    p = float(np.float32(top_p))
    mp = float(np.float32(min_p))
    if k < 0:
        raise ValueError("top_k must be >= 0")
    if not (0.0 < p <= 1.0):
        raise ValueError("top_p must be in (0, 1]")
    if not (0.0 <= mp <= 1.0):
        raise ValueError("min_p must be in [0, 1]")

    n_k = k if 0 < k < V else V

    near_p = False
    if p < 1.0:
        target = p * Z
        hit = np.nonzero(cum >= target)[0]
        r = int(hit[0]) if hit.size else V - 1
        n_p = r + 1
        before = cum[r - 1] if r > 0 else 0.0
        near_p = min(abs(cum[r] - target), abs(target - before)) < MARGIN * Z
    else:
        n_p = V                          # identity: no running sum at all

    near_m = False
    if mp > 0.0:
        thr = math.log(mp)
        gap = s64[pi] - m                # <= 0, non-increasing along pi
        n_m = int(np.count_nonzero(gap >= thr))
        # ln(1) = 0 is exact everywhere; any other threshold carries the
        # rounding of the logarithm.
        scale = MARGIN * max(1.0, abs(thr)) if thr != 0.0 else 0.0
        if n_m > 0 and abs(gap[n_m - 1] - thr) < scale:
            near_m = True
        if n_m < V and abs(gap[n_m] - thr) < scale:
            near_m = True
    else:
        n_m = V

    n = min(n_k, n_p, n_m)
    b = int(pi[n - 1])
    near = (near_p and n_p <= min(n_k, n_m) + 1) or (near_m and n_m <= min(n_k, n_p) + 1)
    return dict(
        n=n, id_thr=b, key_thr=int(order_keys(s[b:b + 1])[0]),
        n_k=n_k, n_p=n_p, n_m=n_m, pi=pi, m=m, Z=Z, mass=cum[n - 1], near=bool(near),
    )


def support(keys: np.ndarray, top_k, top_p, min_p) -> dict:
    """Row-wise support of a [R, V] fp32 key matrix.

    ``top_k``/``top_p``/``min_p`` are per-row arrays (or None for "off").
    Returns arrays ``n``, ``key_thr``, ``id_thr`` (uint32/int64), ``near``,
    and the per-filter prefix lengths ``n_k``, ``n_p``, ``n_m`` (V when the
    filter is off), so a caller can tell which filter binds.
    """
    keys = np.asarray(keys, dtype=np.float32)
    R = keys.shape[0]
    tk, tp, mp = _meta(R, top_k, top_p, min_p)
    n = np.zeros(R, np.int64)
    kt = np.zeros(R, np.uint32)
    it = np.zeros(R, np.int64)
    near = np.zeros(R, bool)
    nk, np_, nm = (np.zeros(R, np.int64) for _ in range(3))
    for r in range(R):
        d = support_row(keys[r], tk[r], tp[r], mp[r])
        n[r], kt[r], it[r], near[r] = d["n"], d["key_thr"], d["id_thr"], d["near"]
        nk[r], np_[r], nm[r] = d["n_k"], d["n_p"], d["n_m"]
    return dict(n=n, key_thr=kt, id_thr=it, near=near, n_k=nk, n_p=np_, n_m=nm)


def binding_filters(sup: dict, V: int) -> dict:
    """Rows on which each filter binds (its prefix is the support; a row may
    count for several filters when their prefixes coincide), and unfiltered
    rows, from the output of ``support``."""
    n = sup["n"]
    out = {"unfiltered": int((n == V).sum())}
    for f, key in (("top_k", "n_k"), ("top_p", "n_p"), ("min_p", "n_m")):
        out[f] = int(((sup[key] == n) & (n < V)).sum())
    return out


def in_support(keys_row: np.ndarray, key_thr: int, id_thr: int) -> np.ndarray:
    """Membership mask from a boundary: key above it, or equal key and id <= it."""
    k = order_keys(keys_row).astype(np.int64)
    ids = np.arange(k.shape[0])
    return (k > key_thr) | ((k == key_thr) & (ids <= id_thr))


def _meta(R, top_k, top_p, min_p):
    tk = np.zeros(R, np.int64) if top_k is None else np.asarray(top_k, np.int64)
    tp = np.ones(R, np.float32) if top_p is None else np.asarray(top_p, np.float32)
    mp = np.zeros(R, np.float32) if min_p is None else np.asarray(min_p, np.float32)
    assert tk.shape == (R,) and tp.shape == (R,) and mp.shape == (R,)
    return tk, tp, mp


# --------------------------------------------------------------------------
# forward and backward
# --------------------------------------------------------------------------
def _logits(h_rows, W, lane, w_scale):
    """The lane's logits of the given rows: fp64 ``h W^T``, or the fp8 lane's
    ``(h8 W8^T) sW a`` (``W`` then holds e4m3 codes)."""
    if lane == "fp8":
        return fp8_logits(h_rows, W, w_scale)
    return chunk_logits(h_rows, W)


def forward(h, W, target, temperature=None, top_k=None, top_p=None, min_p=None,
            keys=None, rows=None, ignore_index=None, lane="fp32", w_scale=None) -> dict:
    """Selected logprob on the filtered support, per row.

    ``h`` [T, H] and ``W`` [V, H] hold the operand values (bf16 or fp32 values,
    any float dtype); ``target`` [T] token ids; metadata per row or None.
    ``keys`` optionally supplies the fp32 keys [len(rows), V] the supports are
    decided on (default: this oracle's own keys).  ``rows`` restricts the
    computation to a subset of rows (all by default).  ``ignore_index``: rows
    whose target equals it are inactive ([nested-learning]
    ``compute_teach_signal``: such rows are masked out of the residual):
    logprob 0 and an exactly zero gradient; their support and side outputs
    are still computed.  ``lane="bf16"``: the bf16 value program (keys from
    ``bf16_lane_keys``, values taken from those keys, logprob rounded to
    bf16); ``lane="fp8"``: ``W`` holds e4m3 codes with per-row scales
    ``w_scale`` and the hidden rows are quantized per row (``fp8_logits``);
    the default is the fp32 program.

    Returns per selected row: ``logprob`` (fp64, -inf out of support),
    ``lse`` (log-sum-exp of z/T over the support), ``n``, ``key_thr``,
    ``id_thr``, ``in_support``, ``near``, and the keys used; and the side
    outputs of one sweep ([align-v2] 5.4 A: the entropy comes out of the
    same pass over the logits):
    ``lse_full`` (log-sum-exp of z/T over the whole row), ``entropy_full``
    (Shannon entropy, in nats, of softmax(z/T) over the whole row) and
    ``entropy_support`` (entropy of the filtered distribution q on the
    support), each ``-sum p log p`` written out term by term.
    """
    h = np.asarray(h)
    T = h.shape[0]
    rows = np.arange(T) if rows is None else np.asarray(rows)
    temp = np.ones(T, np.float32) if temperature is None else np.asarray(temperature, np.float32)
    tk, tp, mp = _meta(T, top_k, top_p, min_p)
    _check_temperature(temp[rows])
    assert lane in ("fp32", "bf16", "fp8"), lane
    z = _logits(h[rows], W, lane, w_scale)                    # fp64 [R, V]
    if keys is not None:
        s32 = canonical_f32(keys)
    elif lane == "bf16":
        s32 = bf16_lane_keys(z, temp[rows])
    else:
        s32 = scale_logits(z, temp[rows])
    # values: fp64 z / T, or in the bf16 lane the bf16 keys themselves
    u = s32.astype(np.float64) if lane == "bf16" else z / temp[rows].astype(np.float64)[:, None]
    R, V = z.shape
    tgt = np.asarray(target, np.int64)[rows]
    ignored = np.zeros(R, bool) if ignore_index is None else tgt == int(ignore_index)
    assert ignore_index is None or not (0 <= int(ignore_index) < V), "ignore_index must not be a token id"
    assert np.all(((tgt >= 0) & (tgt < V)) | ignored), "targets must lie in [0, V)"
    out = dict(logprob=np.empty(R), lse=np.empty(R), n=np.empty(R, np.int64),
               key_thr=np.empty(R, np.uint32), id_thr=np.empty(R, np.int64),
               in_support=np.empty(R, bool), near=np.empty(R, bool), keys=s32,
               rows=rows, lse_full=np.empty(R), entropy_full=np.empty(R), entropy_support=np.empty(R),
               ignored=ignored, lane=lane)
    for i, t in enumerate(rows):
        d = support_row(s32[i], tk[t], tp[t], mp[t])
        S = d["pi"][: d["n"]]
        mx = u[i, S].max()
        lse = mx + math.log(np.exp(u[i, S] - mx).sum())
        inside = bool(np.isin(tgt[i], S)) and not ignored[i]
        lp = 0.0 if ignored[i] else (min(u[i, tgt[i]] - lse, 0.0) if inside else -math.inf)
        if lane == "bf16":
            lp = float(round_to_bf16(np.float32(lp)))             # the lane's logprob dtype
        out["logprob"][i] = lp
        out["lse"][i] = lse
        out["n"][i] = d["n"]
        out["key_thr"][i] = d["key_thr"]
        out["id_thr"][i] = d["id_thr"]
        out["in_support"][i] = inside
        out["near"][i] = d["near"]
        out["lse_full"][i], out["entropy_full"][i] = _entropy(u[i])
        out["entropy_support"][i] = _entropy(u[i, S])[1]
    return out


def _entropy(x) -> tuple:
    """(log-sum-exp, -sum_j p_j log p_j) of the distribution softmax(x)."""
    mx = x.max()
    lse = mx + math.log(np.exp(x - mx).sum())
    logp = x - lse
    return lse, float(-(np.exp(logp) * logp).sum())


def dlogits(h, W, target, fwd: dict, grad_logprob, temperature=None, w_scale=None) -> np.ndarray:
    """``dz[r, j] = g_r (1[j = y_r] - q_rj) / T_r`` on the rows of ``fwd``.

    ``q`` is the softmax of ``z / T`` restricted to the support (in the bf16
    lane of ``fwd``, the softmax of its bf16 keys).  Rows whose target is out
    of support get an exactly zero row whatever ``g`` is.
    """
    rows = fwd["rows"]
    T = np.asarray(h).shape[0]
    temp = np.ones(T, np.float32) if temperature is None else np.asarray(temperature, np.float32)
    lane = fwd.get("lane", "fp32")
    z = _logits(np.asarray(h)[rows], W, lane, w_scale)
    t64 = temp[rows].astype(np.float64)
    u = fwd["keys"].astype(np.float64) if lane == "bf16" else z / t64[:, None]
    g = np.asarray(grad_logprob, np.float64)[rows]
    tgt = np.asarray(target, np.int64)[rows]
    dz = np.zeros_like(z)
    for i in range(len(rows)):
        if not fwd["in_support"][i]:
            continue
        mask = in_support(fwd["keys"][i], int(fwd["key_thr"][i]), int(fwd["id_thr"][i]))
        q = np.where(mask, np.exp(u[i] - fwd["lse"][i]), 0.0)
        onehot = np.zeros_like(q)
        onehot[tgt[i]] = 1.0
        dz[i] = g[i] * (onehot - q) / t64[i]
    return dz


def backward(h, W, target, fwd: dict, grad_logprob, temperature=None, w_scale=None):
    """VJP of ``sum_r g_r * logprob_r`` with respect to ``h`` and ``W``.

    Returns ``(dH, dW)``: ``dH`` [len(rows), H] for the rows of ``fwd`` and
    ``dW`` [V, H] summed over those rows.  In the fp8 lane the quantizations
    pass gradients unchanged (straight through): ``dH = dz W_deq`` and
    ``dW = dz^T h_deq``, the gradients of the product's dequantized operands.
    """
    dz = dlogits(h, W, target, fwd, grad_logprob, temperature, w_scale)
    hr = np.asarray(h)[fwd["rows"]]
    if fwd.get("lane", "fp32") == "fp8":
        W = fp8_dequant_weight(W, w_scale)
        hr = fp8_dequant_rows(hr)
    return gradient_products(dz, hr, W)


def gradient_products(dz, h, W):
    """``(dH, dW) = (dz W, dz^T h)`` in fp64 for ``dz`` [R, V] and the rows
    ``h`` [R, H] it belongs to.  ``dz`` may be a dense array or a
    ``scipy.sparse`` matrix holding the same values (dz is nonzero only on the
    support, so a top-k row has at most k nonzeros): the products are the
    same sums either way."""
    h64 = np.asarray(h, dtype=np.float64)
    W64 = np.asarray(W, dtype=np.float64)
    return np.asarray(dz @ W64), np.asarray(dz.T @ h64)


def round_to_bf16(x) -> np.ndarray:
    """fp32 values rounded to the nearest bf16 (ties to even), as fp32: the
    upper 16 bits of the fp32 pattern after adding 0x7fff plus the lowest
    kept bit (finite inputs)."""
    b = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) & 0xFFFF0000
    return b.astype(np.uint32).view(np.float32)


def bf16_lane_keys(z, temperature) -> np.ndarray:
    """Keys of the bf16 value lane from the logits ``z`` [R, V] (fp64): the
    projection's fp32 value rounded to bf16, divided by the row's temperature
    in fp32 (correctly rounded), and rounded to bf16 again."""
    zb = round_to_bf16(np.asarray(z, np.float64).astype(np.float32))
    return canonical_f32(round_to_bf16(scale_logits(zb, temperature)))


def pre_gemm_hidden(h, temperature, operand="bf16") -> np.ndarray:
    """Scalar pre-GEMM temperature: ``h' = round(fl32(h) / T)`` with the
    quotient correctly rounded to fp32 (an fp64 quotient of fp32 values
    rounded once, as in ``scale_logits``) and then rounded to the operand
    dtype (``"bf16"``, ties to even, or ``"f32"``)."""
    t = np.float32(temperature)
    assert np.isfinite(t) and t > 0, "the scalar temperature must be finite and > 0"
    q = (np.asarray(h, np.float32).astype(np.float64) / np.float64(t)).astype(np.float32)
    return round_to_bf16(q) if operand == "bf16" else q


def backward_pre_gemm(h_scaled, W, target, fwd: dict, grad_logprob, temperature):
    """VJP of ``sum_r g_r * logprob_r`` under the scalar pre-GEMM convention,
    ``fwd`` being ``forward(h_scaled, W, ...)`` with no per-row temperature:
    ``dH = (dz W) / T`` and ``dW = dz^T h_scaled``, ``dz = g (onehot - q)``."""
    dH, dW = backward(h_scaled, W, target, fwd, grad_logprob)
    return dH / float(np.float32(temperature)), dW


# --------------------------------------------------------------------------
# fp8 lm_head lane
# --------------------------------------------------------------------------
# [xorl#74] "What this PR does" 4 rejects FP8 lm_head weights with one
# actionable error; scoring such a head in place of that rejection is read
# here as follows (the pages give no formula).  The weight arrives quantized
# per vocabulary row: e4m3 codes W8 (the OCP "e4m3fn" format: 1 sign, 4
# exponent bits with bias 7, 3 mantissa bits, no infinities, largest finite
# value 448) and one fp32 scale sW[j]: W_deq[j, k] = sW[j] * W8[j, k].
# The hidden states are quantized per row to the same format, so that both
# operands of the product are fp8: a[t] = fl32(max_k |h[t, k]| / 448) (1 for
# an all-zero row) and h8[t, k] = e4m3(clamp(fl32(h[t, k] / a[t]), -448, 448))
# with rounding to nearest, ties to even.  The logits are
# z[t, j] = (sum_k h8[t, k] W8[j, k]) * sW[j] * a[t], the keys and the
# support program follow as in the fp32 lane.  The gradients treat both
# quantizations as identity (straight through): dz as in the fp32 lane, and
# the product's two operands are the dequantized values, so
# dH = dz W_deq and dW = dz^T h_deq with h_deq[t, k] = a[t] h8[t, k] (exact
# products of an fp32 scale and an e4m3 value, kept in fp64 here).

E4M3_MAX = 448.0


def e4m3_encode(x) -> np.ndarray:
    """uint8 e4m3fn codes of fp32 values with |x| <= 448, rounded to nearest
    with ties to even (the format's definition: subnormals m * 2^-9, normals
    (1 + m/8) * 2^(e - 7) for biased exponents e = 1 .. 15)."""
    x = np.asarray(x, np.float32).astype(np.float64)
    assert np.all(np.abs(x) <= E4M3_MAX), "e4m3 input beyond the largest finite value"
    sign = (np.signbit(x)).astype(np.uint32) << 7
    a = np.abs(x)
    out = np.zeros(a.shape, np.uint32)
    sub = a < 2.0 ** -6
    out[sub] = np.rint(a[sub] * 2.0 ** 9).astype(np.uint32)           # 0 .. 8 (8 is the smallest normal)
    nrm = ~sub
    e = np.floor(np.log2(np.where(nrm, a, 1.0))).astype(np.int64)
    q = np.rint(a * np.exp2(3.0 - e))                                   # 8 .. 16, exact scaling
    carry = q == 16.0
    e = np.where(carry, e + 1, e)
    q = np.where(carry, 8.0, q)
    code = ((e + 7) << 3) | (q.astype(np.int64) - 8)
    out[nrm] = code[nrm].astype(np.uint32)
    return (out | sign).astype(np.uint8)


def e4m3_decode(code) -> np.ndarray:
    """fp64 values of e4m3fn codes (0x7F / 0xFF, the NaN codes, are not
    accepted)."""
    c = np.asarray(code, np.uint8).astype(np.int64)
    assert not np.any((c & 0x7F) == 0x7F), "e4m3 NaN code"
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    return sign * mag


def fp8_quantize_rows(h):
    """Per-row quantization of the hidden states: (codes [T, H] uint8,
    scales a [T] fp32) with a = fl32(amax / 448) (1 for a zero row) and
    codes = e4m3(clamp(fl32(h / a), -448, 448))."""
    h32 = np.asarray(h, np.float32)
    amax = np.abs(h32).max(axis=1).astype(np.float64)
    a = np.where(amax > 0, (amax / E4M3_MAX).astype(np.float32), np.float32(1.0)).astype(np.float32)
    x = (h32.astype(np.float64) / a.astype(np.float64)[:, None]).astype(np.float32)
    x = np.clip(x, -E4M3_MAX, E4M3_MAX).astype(np.float32)
    return e4m3_encode(x), a


def fp8_dequant_weight(w8, w_scale) -> np.ndarray:
    """W_deq = sW[j] * W8[j, k] (fp64: the product of an fp32 scale and an
    e4m3 value is exact)."""
    return e4m3_decode(w8) * np.asarray(w_scale, np.float32).astype(np.float64)[:, None]


def fp8_dequant_rows(h) -> np.ndarray:
    """h_deq = a[t] * h8[t, k], the quantized hidden rows' values (fp64,
    exact)."""
    h8, a = fp8_quantize_rows(h)
    return e4m3_decode(h8) * a.astype(np.float64)[:, None]


def fp8_logits(h, w8, w_scale) -> np.ndarray:
    """``z = (h8 W8^T) * sW * a`` in fp64 for the fp8 lane (products of e4m3
    values are exact; the sum is fp64)."""
    h8, a = fp8_quantize_rows(h)
    acc = e4m3_decode(h8) @ e4m3_decode(w8).T
    return acc * np.asarray(w_scale, np.float32).astype(np.float64)[None, :] * a.astype(np.float64)[:, None]


OBJECTIVES = ("cispo", "clip")


def policy_loss(logprob, advantages, old_logprob, objective="cispo", eps_low=0.2, eps_high=0.28,
                scale=1.0) -> dict:
    """Per-token policy-gradient loss and ``g = d loss / d logprob``.

    [align-v2] 5.4 A: the token coefficient ``c`` of ``d loss / d z =
    c (softmax - onehot)`` is ``A sg(clip(r, ., 1 + eps_high))`` for CISPO
    (the importance weight is a stop-gradient constant, with no lower clip)
    and ``A r 1[not clipped]`` for the clipped surrogate (clip-higher
    PPO/DAPO), both in the loss sign; ``d logprob / d z = onehot - softmax``,
    so ``g = -c``.  The losses are the functions with those derivatives:
    ``-A sg(w) logprob`` and ``-min(r A, clip(r, 1 - eps_low, 1 + eps_high) A)``.

    A row whose logprob is -inf (target outside the support) has no
    defined ratio; it contributes zero loss and zero gradient, like the
    logprob's own gradient on such rows.  A NaN logprob (invalid row)
    gives a NaN loss and zero gradient.  Everything is multiplied by
    ``scale``.  Returns ``loss``, ``g`` and ``ratio`` (fp64 arrays).
    """
    if objective not in OBJECTIVES:
        raise ValueError(f"objective must be one of {OBJECTIVES}")
    lp = np.asarray(logprob, np.float64)
    A = np.asarray(advantages, np.float32).astype(np.float64)
    old = np.asarray(old_logprob, np.float32).astype(np.float64)
    eh = float(np.float32(eps_high))
    el = float(np.float32(eps_low))
    sc = float(np.float32(scale))
    loss = np.zeros_like(lp)
    g = np.zeros_like(lp)
    ratio = np.zeros_like(lp)
    for t in range(lp.shape[0]):
        if math.isnan(lp[t]):
            loss[t] = math.nan
            continue
        if lp[t] == -math.inf:
            continue
        r = math.exp(lp[t] - old[t])
        ratio[t] = r
        if objective == "cispo":
            wgt = min(r, 1.0 + eh)
            loss[t] = -A[t] * wgt * lp[t]
            g[t] = -A[t] * wgt
        else:
            unclipped = r * A[t]
            clipped = min(max(r, 1.0 - el), 1.0 + eh) * A[t]
            if unclipped <= clipped:
                loss[t] = -unclipped
                g[t] = -A[t] * r
            else:
                loss[t] = -clipped
                g[t] = 0.0
    return dict(loss=loss * sc, g=g * sc, ratio=ratio)


def sample_targets(h, W, temperature, top_k, top_p, min_p, u, rows=None, lane="fp32", w_scale=None) -> np.ndarray:
    """Draw one target per row from its filtered distribution.

    Inverse CDF along the order pi over ``q`` (softmax of z/T on the
    support), with the caller's uniforms ``u`` in [0, 1).  ``rows`` limits
    the draw to a subset of rows (returned in that order).  ``lane="fp8"``
    takes the fp8 lane's logits (``W`` of e4m3 codes, row scales
    ``w_scale``).
    """
    T = np.asarray(h).shape[0]
    rows = np.arange(T) if rows is None else np.asarray(rows)
    temp = np.ones(T, np.float32) if temperature is None else np.asarray(temperature, np.float32)
    tk, tp, mp = _meta(T, top_k, top_p, min_p)
    z = _logits(np.asarray(h)[rows], W, "fp8" if lane == "fp8" else "fp32", w_scale)
    s32 = scale_logits(z, temp[rows])
    uu = z / temp[rows].astype(np.float64)[:, None]
    out = np.empty(len(rows), np.int64)
    for i, t in enumerate(rows):
        d = support_row(s32[i], tk[t], tp[t], mp[t])
        S = d["pi"][: d["n"]]
        w = np.exp(uu[i, S] - uu[i, S].max())
        cdf = np.cumsum(w)
        j = int(np.searchsorted(cdf, float(u[t]) * cdf[-1], side="right"))
        out[i] = S[min(j, len(S) - 1)]
    return out


def _check_temperature(t):
    t = np.asarray(t, np.float32)
    if not np.all(np.isfinite(t) & (t > 0)):
        raise ValueError("temperature must be finite and > 0")
