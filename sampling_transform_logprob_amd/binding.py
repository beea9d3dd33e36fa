"""ctypes binding of ``libstce.so`` (argument marshalling only).

Every step of the scoring path runs in the HIP library; this module checks
tensor shapes/dtypes/devices, allocates outputs and workspaces with torch and
passes raw device pointers plus the current HIP stream to the C ABI declared
in ``include/stce.h``.  There is no fallback: without the built library every
entry point raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libstce.so")

STATUS_NONE = (1 << 63) - 1
FIELDS = {1: "temperature", 2: "top_k", 3: "top_p", 4: "min_p", 5: "target"}
FLAG_VALID, FLAG_FILTERED, FLAG_IN_SUPPORT, FLAG_IGNORED, FLAG_LISTED = 1, 2, 4, 8, 32
PROBLEM_IGNORE_INDEX, PROBLEM_PRE_GEMM_TEMPERATURE, PROBLEM_BF16_LANE, PROBLEM_RECOMPUTE_ALL = 1, 2, 4, 8
LANES = {"fp32": 0, "bf16": PROBLEM_BF16_LANE}
# a 32-byte record, then (after all T records) a 64-byte tile list, then a
# support list of NSP (token id, key) pairs
RECORD_BYTES = 32
NTILE = 31
NSP = 128
STATE_BYTES_PER_ROW = RECORD_BYTES + 2 * (1 + NTILE) + 8 * NSP
DT_BF16, DT_F32, DT_FP8 = 1, 2, 3
# dtypes a weight of e4m3 codes may come in (the fp8 lane)
FP8_WEIGHT_DTYPES = (torch.uint8, torch.float8_e4m3fn)

SYMBOLS = (
    "stce_state_bytes", "stce_workspace_bytes", "stce_forward", "stce_backward",
    "stce_scaled_logits", "stce_support_from_logits", "stce_support_workspace_bytes",
    "stce_decode_state", "stce_status_string", "stce_last_error", "stce_profile_attach", "stce_schedule",
    "stce_policy_loss", "stce_forward_with_side", "stce_fused_workspace_bytes", "stce_fused_policy_step",
    "stce_recompute_keys", "stce_forward_noalloc", "stce_noalloc_scratch_bytes", "stce_fp8_quantize_rows",
)
KERNEL_KINDS = {1: "validate", 2: "projection", 3: "select", 4: "dlogits", 5: "grad_weight",
                6: "grad_hidden", 7: "transpose", 8: "partials", 9: "policy_loss", 10: "dz_keys",
                11: "split_sum", 12: "prescale", 13: "classify", 14: "sparse_grad_weight",
                15: "sparse_grad_hidden", 16: "reproject", 17: "quantize", 18: "tile_lists",
                19: "tile_recompute", 20: "listed_entries"}
PG_OBJECTIVES = {"cispo": 1, "clip": 2}


class Problem(ctypes.Structure):
    _fields_ = [
        ("T", ctypes.c_int64), ("H", ctypes.c_int64), ("V", ctypes.c_int64),
        ("dtype", ctypes.c_int32), ("flags", ctypes.c_int32),
        ("hidden", ctypes.c_void_p), ("weight", ctypes.c_void_p), ("target", ctypes.c_void_p),
        ("temperature", ctypes.c_void_p), ("top_k", ctypes.c_void_p), ("top_p", ctypes.c_void_p),
        ("min_p", ctypes.c_void_p), ("chunk_rows", ctypes.c_int64), ("vocab_slice", ctypes.c_int64),
        ("ignore_index", ctypes.c_int64), ("pre_gemm_temperature", ctypes.c_float),
        ("weight_scale", ctypes.c_void_p),
    ]


class RowInfo(ctypes.Structure):
    _fields_ = [
        ("key_thr", ctypes.c_uint32), ("id_thr", ctypes.c_int32), ("n", ctypes.c_int32),
        ("flags", ctypes.c_uint32), ("lse_support", ctypes.c_float), ("lse_full", ctypes.c_float),
        ("row_max", ctypes.c_float), ("target_key", ctypes.c_float),
    ]


class Profile(ctypes.Structure):
    _fields_ = [("capacity", ctypes.c_int32), ("count", ctypes.c_int32),
                ("start", ctypes.POINTER(ctypes.c_void_p)), ("stop", ctypes.POINTER(ctypes.c_void_p)),
                ("kind", ctypes.POINTER(ctypes.c_int32))]


class PgParams(ctypes.Structure):
    _fields_ = [
        ("objective", ctypes.c_int32), ("eps_low", ctypes.c_float), ("eps_high", ctypes.c_float),
        ("scale", ctypes.c_float), ("advantages", ctypes.c_void_p), ("old_logprob", ctypes.c_void_p),
        ("state", ctypes.c_void_p),
    ]


class SideOutputs(ctypes.Structure):
    _fields_ = [("lse_full", ctypes.c_void_p), ("entropy_full", ctypes.c_void_p),
                ("entropy_support", ctypes.c_void_p)]


class StceError(RuntimeError):
    pass


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the HIP library (once) and declare its signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise StceError(f"{path} is not built: run sampling_transform_logprob_amd/build.py")
    L = ctypes.CDLL(path)
    P, vp, i64, i32, sz = ctypes.POINTER(Problem), ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
    sig = {
        "stce_state_bytes": (sz, [i64]),
        "stce_workspace_bytes": (ctypes.c_int, [P, ctypes.POINTER(sz), ctypes.POINTER(sz)]),
        "stce_forward": (ctypes.c_int, [P, vp, vp, vp, vp, sz, vp]),
        "stce_backward": (ctypes.c_int, [P, vp, vp, vp, vp, i32, vp, vp, sz, vp]),
        "stce_recompute_keys": (ctypes.c_int, [P, vp, vp, vp, vp, sz, vp]),
        "stce_forward_noalloc": (ctypes.c_int, [P, vp, vp, vp, vp]),
        "stce_noalloc_scratch_bytes": (sz, []),
        "stce_fp8_quantize_rows": (ctypes.c_int, [vp, i64, i64, vp, vp, vp]),
        "stce_scaled_logits": (ctypes.c_int, [P, i64, i64, vp, vp, sz, vp]),
        "stce_support_from_logits": (ctypes.c_int, [vp, i64, i64, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
        "stce_support_workspace_bytes": (sz, [i64, i64]),
        "stce_decode_state": (ctypes.c_int, [vp, i64, ctypes.POINTER(RowInfo)]),
        "stce_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "stce_last_error": (ctypes.c_char_p, []),
        "stce_profile_attach": (ctypes.c_int, [ctypes.POINTER(Profile)]),
        "stce_schedule": (ctypes.c_int, [P, ctypes.POINTER(i64), ctypes.POINTER(i64)]),
        "stce_policy_loss": (ctypes.c_int, [ctypes.POINTER(PgParams), i64, vp, vp, vp, vp, vp]),
        "stce_forward_with_side": (ctypes.c_int, [P, vp, vp, ctypes.POINTER(SideOutputs), vp, vp, sz, vp]),
        "stce_fused_workspace_bytes": (ctypes.c_int, [P, ctypes.POINTER(sz), ctypes.POINTER(sz)]),
        "stce_fused_policy_step": (ctypes.c_int, [P, ctypes.POINTER(PgParams), vp, vp, vp, vp,
                                                  ctypes.POINTER(SideOutputs), vp, vp, i32, vp, vp, sz, vp]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype, f.argtypes = res, args
    _lib = L
    return L


def _check(status: int) -> None:
    if status != 0:
        L = load()
        raise StceError(f"{L.stce_status_string(status).decode()}: {L.stce_last_error().decode()}")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream() -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _meta(name, t, T, dtype, device):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor or None")
    if t.dim() != 1 or t.shape[0] != T:
        # over-length (or short) per-row metadata is an error, never truncated
        raise ValueError(f"{name} must have shape [{T}], got {tuple(t.shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    return t.contiguous()


def make_problem(hidden, weight, target, temperature=None, top_k=None, top_p=None, min_p=None,
                 chunk_rows: int = 0, vocab_slice: int = 0, ignore_index: Optional[int] = None,
                 pre_gemm_temperature: Optional[float] = None, lane: str = "fp32",
                 weight_scale: Optional[torch.Tensor] = None, recompute_all: bool = False):
    """Checked ``stce_problem`` plus the tensors it points into (kept alive).

    ``temperature`` is the per-row tensor applied to the logits after the
    product; ``pre_gemm_temperature`` is instead one scalar applied to the
    hidden states before it (the two do not combine).  ``lane="bf16"`` runs
    the bf16 value program (bf16 keys; the logprob, still an fp32 tensor,
    holds bf16 values, so ``.bfloat16()`` is exact).  A weight of e4m3 codes
    (``torch.uint8`` or ``torch.float8_e4m3fn``) with ``weight_scale`` (fp32
    [V]) and bf16 hidden states selects the fp8 lane."""
    if lane not in LANES:
        raise ValueError(f"lane must be one of {tuple(LANES)}")
    if pre_gemm_temperature is not None and temperature is not None:
        raise ValueError("pass either a per-row temperature tensor or pre_gemm_temperature, not both")
    if hidden.dim() != 2 or weight.dim() != 2 or hidden.shape[1] != weight.shape[1]:
        raise ValueError(f"hidden [T, H] and weight [V, H] expected, got {tuple(hidden.shape)}, {tuple(weight.shape)}")
    if weight.dtype in FP8_WEIGHT_DTYPES:
        if hidden.dtype != torch.bfloat16:
            raise TypeError(f"the fp8 lane takes bf16 hidden states, got {hidden.dtype}")
        if weight_scale is None:
            raise ValueError("an e4m3 weight needs weight_scale (fp32 [V])")
        dt = DT_FP8
        weight = weight.view(torch.uint8)
    else:
        if weight_scale is not None:
            raise ValueError("weight_scale is for an e4m3 weight only")
        if hidden.dtype != weight.dtype:
            raise TypeError(f"hidden ({hidden.dtype}) and weight ({weight.dtype}) must share a dtype")
        dt = {torch.bfloat16: DT_BF16, torch.float32: DT_F32}.get(hidden.dtype)
        if dt is None:
            raise TypeError(
                f"unsupported LM-head dtype {hidden.dtype}: scoring takes bf16 or fp32 hidden/weight, or an "
                "e4m3 weight with per-row scales (the fp8 lane)")
    if hidden.device.type != "cuda" or weight.device != hidden.device:
        raise ValueError("hidden and weight must be on the same GPU")
    T, H = hidden.shape
    V = weight.shape[0]
    dev = hidden.device
    hidden, weight = hidden.contiguous(), weight.contiguous()
    if weight_scale is not None:
        weight_scale = _meta("weight_scale", weight_scale, V, torch.float32, dev)
    target = _meta("target", target, T, torch.int64, dev)
    if target is None:
        raise ValueError("target is required")
    keep = [hidden, weight, target,
            _meta("temperature", temperature, T, torch.float32, dev),
            _meta("top_k", top_k, T, torch.int32, dev),
            _meta("top_p", top_p, T, torch.float32, dev),
            _meta("min_p", min_p, T, torch.float32, dev)]
    flags = (0 if ignore_index is None else PROBLEM_IGNORE_INDEX) | LANES[lane]
    if pre_gemm_temperature is not None:
        flags |= PROBLEM_PRE_GEMM_TEMPERATURE
    if recompute_all:
        flags |= PROBLEM_RECOMPUTE_ALL
    prob = Problem(T, H, V, dt, flags, *[t.data_ptr() if t is not None else None for t in keep], chunk_rows,
                   vocab_slice, 0 if ignore_index is None else int(ignore_index),
                   0.0 if pre_gemm_temperature is None else float(pre_gemm_temperature),
                   None if weight_scale is None else weight_scale.data_ptr())
    keep.append(weight_scale)
    return prob, keep


def workspace_bytes(prob: Problem):
    f, b = ctypes.c_size_t(), ctypes.c_size_t()
    _check(load().stce_workspace_bytes(ctypes.byref(prob), ctypes.byref(f), ctypes.byref(b)))
    return f.value, b.value


def schedule(prob: Problem):
    """(forward rows per chunk, backward vocabulary columns per slice)."""
    c, v = ctypes.c_int64(), ctypes.c_int64()
    _check(load().stce_schedule(ctypes.byref(prob), ctypes.byref(c), ctypes.byref(v)))
    return c.value, v.value


def _raise_rows(status: torch.Tensor, what: str, tensors: dict) -> None:
    v = int(status.item())
    if v == STATUS_NONE:
        return
    row, field = v >> 8, v & 0xFF
    name = FIELDS.get(field, f"field {field}")
    t = tensors.get(name)
    val = "" if t is None else f"={t[row].item()!r}"
    raise ValueError(f"{what}: invalid {name}[{row}]{val}")


def forward(hidden, weight, target, temperature=None, top_k=None, top_p=None, min_p=None, *,
            chunk_rows: int = 0, check: bool = True, workspace: Optional[torch.Tensor] = None,
            side: bool = False, ignore_index: Optional[int] = None, pre_gemm_temperature: Optional[float] = None,
            lane: str = "fp32", weight_scale: Optional[torch.Tensor] = None):
    """Selected logprob per row and the per-row state for backward.

    With ``side=True`` also returns a dict of the sweep's side outputs
    (``lse_full``, ``entropy_full``, ``entropy_support``, fp32 [T]).
    """
    prob, keep = make_problem(hidden, weight, target, temperature, top_k, top_p, min_p, chunk_rows,
                              ignore_index=ignore_index, pre_gemm_temperature=pre_gemm_temperature, lane=lane,
                              weight_scale=weight_scale)
    T = prob.T
    fwd_b, _ = workspace_bytes(prob)
    dev = hidden.device
    ws = workspace if workspace is not None else torch.empty(max(fwd_b, 1), dtype=torch.uint8, device=dev)
    logprob = torch.empty(T, dtype=torch.float32, device=dev)
    state = torch.empty(T * STATE_BYTES_PER_ROW, dtype=torch.uint8, device=dev)
    status = torch.empty(1, dtype=torch.int64, device=dev)
    outs = None
    if side:
        outs = {k: torch.empty(T, dtype=torch.float32, device=dev)
                for k in ("lse_full", "entropy_full", "entropy_support")}
        so = SideOutputs(*(outs[k].data_ptr() for k in ("lse_full", "entropy_full", "entropy_support")))
        _check(load().stce_forward_with_side(ctypes.byref(prob), _ptr(logprob), _ptr(state), ctypes.byref(so),
                                             _ptr(status), _ptr(ws), ws.numel(), _stream()))
    else:
        _check(load().stce_forward(ctypes.byref(prob), _ptr(logprob), _ptr(state), _ptr(status), _ptr(ws),
                                   ws.numel(), _stream()))
    if check:
        _raise_rows(status, "stce_forward", dict(temperature=keep[3], top_k=keep[4], top_p=keep[5],
                                                 min_p=keep[6], target=keep[2]))
    return (logprob, state, outs) if side else (logprob, state)


def forward_noalloc(hidden, weight, target, temperature=None, top_k=None, top_p=None, min_p=None, *,
                    chunk_rows: int = 0, check: bool = True, ignore_index: Optional[int] = None,
                    pre_gemm_temperature: Optional[float] = None, lane: str = "fp32",
                    weight_scale: Optional[torch.Tensor] = None):
    """``forward`` through ``stce_forward_noalloc``: the library's static
    scratch instead of a workspace (the outputs are still allocated here)."""
    prob, keep = make_problem(hidden, weight, target, temperature, top_k, top_p, min_p, chunk_rows,
                              ignore_index=ignore_index, pre_gemm_temperature=pre_gemm_temperature, lane=lane,
                              weight_scale=weight_scale)
    T = prob.T
    dev = hidden.device
    logprob = torch.empty(T, dtype=torch.float32, device=dev)
    state = torch.empty(T * STATE_BYTES_PER_ROW, dtype=torch.uint8, device=dev)
    status = torch.empty(1, dtype=torch.int64, device=dev)
    _check(load().stce_forward_noalloc(ctypes.byref(prob), _ptr(logprob), _ptr(state), _ptr(status), _stream()))
    if check:
        _raise_rows(status, "stce_forward_noalloc", dict(temperature=keep[3], top_k=keep[4], top_p=keep[5],
                                                         min_p=keep[6], target=keep[2]))
    return logprob, state


def backward(hidden, weight, target, state, grad_logprob, temperature=None, top_k=None, top_p=None,
             min_p=None, *, need_hidden: bool = True, need_weight: bool = True,
             grad_weight: Optional[torch.Tensor] = None, accumulate_grad_weight: bool = False,
             vocab_slice: int = 0, workspace: Optional[torch.Tensor] = None, ignore_index: Optional[int] = None,
             pre_gemm_temperature: Optional[float] = None, lane: str = "fp32",
             weight_scale: Optional[torch.Tensor] = None, recompute_all: bool = False):
    """(grad_hidden [T, H] in hidden's dtype, grad_weight [V, H] fp32).
    ``recompute_all`` recomputes every row's keys, ignoring the support
    lists the state holds."""
    prob, keep = make_problem(hidden, weight, target, temperature, top_k, top_p, min_p, 0, vocab_slice,
                              ignore_index=ignore_index, pre_gemm_temperature=pre_gemm_temperature, lane=lane,
                              weight_scale=weight_scale, recompute_all=recompute_all)
    T, H, V = prob.T, prob.H, prob.V
    dev = hidden.device
    if grad_logprob.shape != (T,) or grad_logprob.dtype != torch.float32 or grad_logprob.device != dev:
        raise ValueError("grad_logprob must be fp32 [T] on the hidden's device")
    if state.numel() != T * STATE_BYTES_PER_ROW or state.dtype != torch.uint8:
        raise ValueError(f"state must be the uint8 [T*{STATE_BYTES_PER_ROW}] tensor written by forward")
    g = grad_logprob.contiguous()
    _, bwd_b = workspace_bytes(prob)
    ws = workspace if workspace is not None else torch.empty(max(bwd_b, 1), dtype=torch.uint8, device=dev)
    gh = torch.empty(T, H, dtype=hidden.dtype, device=dev) if need_hidden else None
    if need_weight:
        if grad_weight is None:
            grad_weight = torch.empty(V, H, dtype=torch.float32, device=dev)
            accumulate_grad_weight = False
        elif grad_weight.shape != (V, H) or grad_weight.dtype != torch.float32 or not grad_weight.is_contiguous():
            raise ValueError("grad_weight must be a contiguous fp32 [V, H] tensor")
    else:
        grad_weight = None
    _check(load().stce_backward(ctypes.byref(prob), _ptr(g), _ptr(state), _ptr(gh), _ptr(grad_weight),
                                1 if accumulate_grad_weight else 0, None, _ptr(ws), ws.numel(), _stream()))
    return gh, grad_weight


def recompute_keys(hidden, weight, target, state, grad_logprob, temperature=None, top_k=None, top_p=None,
                   min_p=None, *, vocab_slice: int = 0, ignore_index: Optional[int] = None,
                   pre_gemm_temperature: Optional[float] = None, lane: str = "fp32",
                   weight_scale: Optional[torch.Tensor] = None):
    """fp32 keys [T, V] recomputed by the backward's products, exported by
    those launches themselves (parity: they must equal the forward's bit for
    bit).  A row whose keys the backward recomputes on its listed tiles only
    gets those tiles' keys; its other entries stay NaN."""
    prob, keep = make_problem(hidden, weight, target, temperature, top_k, top_p, min_p, 0, vocab_slice,
                              ignore_index=ignore_index, pre_gemm_temperature=pre_gemm_temperature, lane=lane,
                              weight_scale=weight_scale)
    dev = hidden.device
    if state.numel() != prob.T * STATE_BYTES_PER_ROW or state.dtype != torch.uint8:
        raise ValueError(f"state must be the uint8 [T*{STATE_BYTES_PER_ROW}] tensor written by forward")
    _, bwd_b = workspace_bytes(prob)
    ws = torch.empty(max(bwd_b, 1), dtype=torch.uint8, device=dev)
    out = torch.full((prob.T, prob.V), float("nan"), dtype=torch.float32, device=dev)
    g = grad_logprob.contiguous()
    _check(load().stce_recompute_keys(ctypes.byref(prob), _ptr(g), _ptr(state), _ptr(out), _ptr(ws), ws.numel(),
                                      _stream()))
    return out


def scaled_logits(hidden, weight, temperature=None, row0: int = 0, nrows: Optional[int] = None, *,
                  pre_gemm_temperature: Optional[float] = None, lane: str = "fp32",
                  weight_scale: Optional[torch.Tensor] = None):
    """fp32 keys of rows [row0, row0 + nrows) from the forward's kernel:
    s = fl32(h W^T) / T per row, or fl32((h / Ts) W^T) with the scalar
    pre-GEMM temperature Ts; in the bf16 lane the bf16 keys."""
    T = hidden.shape[0]
    nrows = T - row0 if nrows is None else nrows
    target = torch.zeros(T, dtype=torch.int64, device=hidden.device)
    prob, keep = make_problem(hidden, weight, target, temperature, pre_gemm_temperature=pre_gemm_temperature,
                              lane=lane, weight_scale=weight_scale)
    fwd_b, _ = workspace_bytes(prob)
    ws = torch.empty(max(fwd_b, 1), dtype=torch.uint8, device=hidden.device)
    out = torch.empty(nrows, prob.V, dtype=torch.float32, device=hidden.device)
    _check(load().stce_scaled_logits(ctypes.byref(prob), row0, nrows, _ptr(out), _ptr(ws), ws.numel(), _stream()))
    return out


def fp8_quantize_rows(x: torch.Tensor):
    """(codes uint8 [R, H], scales fp32 [R]): the fp8 lane's per-row e4m3
    quantization of bf16 rows ``x`` [R, H] (H a multiple of 16)."""
    if x.dim() != 2 or x.dtype != torch.bfloat16 or x.device.type != "cuda":
        raise ValueError("x must be a bf16 [R, H] tensor on a GPU")
    x = x.contiguous()
    R, H = x.shape
    codes = torch.empty(R, H, dtype=torch.uint8, device=x.device)
    scales = torch.empty(R, dtype=torch.float32, device=x.device)
    _check(load().stce_fp8_quantize_rows(_ptr(x), R, H, _ptr(codes), _ptr(scales), _stream()))
    return codes, scales


def support_from_logits(s, target, top_k=None, top_p=None, min_p=None, *, check: bool = True):
    """Support program + selected logprob on given fp32 keys s [R, V]."""
    if s.dim() != 2 or s.dtype != torch.float32 or s.device.type != "cuda":
        raise ValueError("s must be a fp32 [R, V] GPU tensor")
    s = s.contiguous()
    R, V = s.shape
    dev = s.device
    target = _meta("target", target, R, torch.int64, dev)
    tk = _meta("top_k", top_k, R, torch.int32, dev)
    tp = _meta("top_p", top_p, R, torch.float32, dev)
    mp = _meta("min_p", min_p, R, torch.float32, dev)
    L = load()
    nb = L.stce_support_workspace_bytes(R, V)
    ws = torch.empty(max(nb, 1), dtype=torch.uint8, device=dev)
    logprob = torch.empty(R, dtype=torch.float32, device=dev)
    state = torch.empty(R * STATE_BYTES_PER_ROW, dtype=torch.uint8, device=dev)
    status = torch.empty(1, dtype=torch.int64, device=dev)
    _check(L.stce_support_from_logits(_ptr(s), R, V, _ptr(tk), _ptr(tp), _ptr(mp), _ptr(target), _ptr(logprob),
                                      _ptr(state), _ptr(status), _ptr(ws), ws.numel(), _stream()))
    if check:
        _raise_rows(status, "stce_support_from_logits", dict(top_k=tk, top_p=tp, min_p=mp, target=target))
    return logprob, state


def policy_loss(logprob, advantages, old_logprob, objective: str = "cispo", eps_low: float = 0.2,
                eps_high: float = 0.28, scale: float = 1.0, state: Optional[torch.Tensor] = None):
    """Per-token policy-gradient loss on the selected logprob.

    Returns (loss [T], grad_logprob [T], ratio [T]); grad_logprob is the
    upstream gradient to pass to ``backward`` for d(sum loss)/d(h, W).
    """
    if objective not in PG_OBJECTIVES:
        raise ValueError(f"objective must be one of {tuple(PG_OBJECTIVES)}")
    if logprob.dim() != 1 or logprob.dtype != torch.float32:
        raise ValueError("logprob must be fp32 [T]")
    T = logprob.shape[0]
    dev = logprob.device
    adv = _meta("advantages", advantages, T, torch.float32, dev)
    old = _meta("old_logprob", old_logprob, T, torch.float32, dev)
    if adv is None or old is None:
        raise ValueError("advantages and old_logprob are required")
    lp = logprob.contiguous()
    loss = torch.empty(T, dtype=torch.float32, device=dev)
    grad = torch.empty(T, dtype=torch.float32, device=dev)
    ratio = torch.empty(T, dtype=torch.float32, device=dev)
    pg = PgParams(PG_OBJECTIVES[objective], eps_low, eps_high, scale, adv.data_ptr(), old.data_ptr(),
                  None if state is None else state.data_ptr())
    _check(load().stce_policy_loss(ctypes.byref(pg), T, _ptr(lp), _ptr(loss), _ptr(grad), _ptr(ratio), _stream()))
    return loss, grad, ratio


def policy_loss_step(hidden, weight, target, advantages, old_logprob, temperature=None, top_k=None, top_p=None,
                     min_p=None, *, objective: str = "cispo", eps_low: float = 0.2, eps_high: float = 0.28,
                     scale: float = 1.0, need_hidden: bool = True, need_weight: bool = True,
                     ignore_index: Optional[int] = None, pre_gemm_temperature: Optional[float] = None,
                     lane: str = "fp32"):
    """Fused head + policy-gradient token loss: forward, per-token loss and
    the gradients of ``sum(loss)``.  Returns (loss [T], logprob [T], ratio [T],
    grad_hidden, grad_weight)."""
    logprob, state = forward(hidden, weight, target, temperature, top_k, top_p, min_p, ignore_index=ignore_index,
                             pre_gemm_temperature=pre_gemm_temperature, lane=lane)
    loss, g, ratio = policy_loss(logprob, advantages, old_logprob, objective, eps_low, eps_high, scale, state)
    gh, gw = backward(hidden, weight, target, state, g, temperature, top_k, top_p, min_p,
                      need_hidden=need_hidden, need_weight=need_weight, ignore_index=ignore_index,
                      pre_gemm_temperature=pre_gemm_temperature, lane=lane)
    return loss, logprob, ratio, gh, gw


def fused_workspace_bytes(prob: Problem):
    """(default, minimum) workspace bytes of the fused step; a size between
    them keeps fewer chunks per weight-gradient group."""
    n, m = ctypes.c_size_t(), ctypes.c_size_t()
    _check(load().stce_fused_workspace_bytes(ctypes.byref(prob), ctypes.byref(n), ctypes.byref(m)))
    return n.value, m.value


def fused_policy_step(hidden, weight, target, advantages, old_logprob, temperature=None, top_k=None, top_p=None,
                      min_p=None, *, objective: str = "cispo", eps_low: float = 0.2, eps_high: float = 0.28,
                      scale: float = 1.0, need_hidden: bool = True, need_weight: bool = True,
                      grad_weight: Optional[torch.Tensor] = None, accumulate_grad_weight: bool = False,
                      side: bool = False, chunk_rows: int = 0, ignore_index: Optional[int] = None,
                      check: bool = True, workspace: Optional[torch.Tensor] = None,
                      pre_gemm_temperature: Optional[float] = None, lane: str = "fp32",
                      weight_scale: Optional[torch.Tensor] = None, recompute_all: bool = False):
    """The fused head + policy-gradient step (dlogits formed in the forward's
    sweep from the chunk's keys).  Returns a dict with ``loss``, ``logprob``,
    ``ratio`` (fp32 [T]), ``state``, ``grad_hidden`` ([T, H], hidden's dtype,
    or None), ``grad_weight`` (fp32 [V, H] or None) and, with ``side=True``,
    ``lse_full``, ``entropy_full``, ``entropy_support``.  An e4m3 ``weight``
    (uint8 codes) with ``weight_scale`` takes the fp8 lane."""
    if objective not in PG_OBJECTIVES:
        raise ValueError(f"objective must be one of {tuple(PG_OBJECTIVES)}")
    prob, keep = make_problem(hidden, weight, target, temperature, top_k, top_p, min_p, chunk_rows,
                              ignore_index=ignore_index, pre_gemm_temperature=pre_gemm_temperature, lane=lane,
                              weight_scale=weight_scale, recompute_all=recompute_all)
    T, H, V = prob.T, prob.H, prob.V
    dev = hidden.device
    adv = _meta("advantages", advantages, T, torch.float32, dev)
    old = _meta("old_logprob", old_logprob, T, torch.float32, dev)
    if adv is None or old is None:
        raise ValueError("advantages and old_logprob are required")
    keep += [adv, old]
    nb, _ = fused_workspace_bytes(prob)
    ws = workspace if workspace is not None else torch.empty(max(nb, 1), dtype=torch.uint8, device=dev)
    out = {k: torch.empty(T, dtype=torch.float32, device=dev) for k in ("loss", "logprob", "ratio")}
    out["state"] = torch.empty(T * STATE_BYTES_PER_ROW, dtype=torch.uint8, device=dev)
    out["grad_hidden"] = torch.empty(T, H, dtype=hidden.dtype, device=dev) if need_hidden else None
    if need_weight:
        if grad_weight is None:
            grad_weight = torch.empty(V, H, dtype=torch.float32, device=dev)
            accumulate_grad_weight = False
        elif grad_weight.shape != (V, H) or grad_weight.dtype != torch.float32 or not grad_weight.is_contiguous():
            raise ValueError("grad_weight must be a contiguous fp32 [V, H] tensor")
    else:
        grad_weight = None
    out["grad_weight"] = grad_weight
    so = None
    if side:
        for k in ("lse_full", "entropy_full", "entropy_support"):
            out[k] = torch.empty(T, dtype=torch.float32, device=dev)
        so = SideOutputs(*(out[k].data_ptr() for k in ("lse_full", "entropy_full", "entropy_support")))
    pg = PgParams(PG_OBJECTIVES[objective], eps_low, eps_high, scale, adv.data_ptr(), old.data_ptr(), None)
    status = torch.empty(1, dtype=torch.int64, device=dev)
    _check(load().stce_fused_policy_step(ctypes.byref(prob), ctypes.byref(pg), _ptr(out["logprob"]),
                                         _ptr(out["state"]), _ptr(out["loss"]), _ptr(out["ratio"]),
                                         None if so is None else ctypes.byref(so), _ptr(out["grad_hidden"]),
                                         _ptr(grad_weight), 1 if accumulate_grad_weight else 0, _ptr(status),
                                         _ptr(ws), ws.numel(), _stream()))
    if check:
        _raise_rows(status, "stce_fused_policy_step", dict(temperature=keep[3], top_k=keep[4], top_p=keep[5],
                                                            min_p=keep[6], target=keep[2]))
    return out


def decode_state(state: torch.Tensor) -> dict:
    """Per-row state fields as numpy arrays (copies the state to the host),
    with ``ntile`` and ``tiles`` [T, 31] from the rows' tile lists, and
    ``support_ids`` / ``support_keys`` [T, 128] from their support lists."""
    import numpy as np
    host = state.detach().cpu().contiguous()
    n = host.numel() // STATE_BYTES_PER_ROW
    out = (RowInfo * n)()
    _check(load().stce_decode_state(ctypes.c_void_p(host.data_ptr()), n, out))
    arr = np.frombuffer(bytes(out), dtype=np.dtype([
        ("key_thr", "<u4"), ("id_thr", "<i4"), ("n", "<i4"), ("flags", "<u4"),
        ("lse_support", "<f4"), ("lse_full", "<f4"), ("row_max", "<f4"), ("target_key", "<f4")]))
    d = {k: arr[k].copy() for k in arr.dtype.names}
    tb = 2 * (1 + NTILE)
    tl = host[n * RECORD_BYTES:n * (RECORD_BYTES + tb)].numpy().view(np.uint16).reshape(n, 1 + NTILE)
    d["ntile"] = tl[:, 0].astype(np.int64)
    d["tiles"] = tl[:, 1:].astype(np.int64)
    sl = host[n * (RECORD_BYTES + tb):].numpy().view(np.int32).reshape(n, NSP, 2)
    d["support_ids"] = sl[:, :, 0].astype(np.int64)
    d["support_keys"] = sl[:, :, 1].copy().view(np.float32)
    return d


def state_prefix(state: torch.Tensor, rows: int) -> torch.Tensor:
    """The state bytes of the first ``rows`` rows (their records, their tile
    lists, then their support lists), comparable with the state of a call
    over those rows only."""
    T = state.numel() // STATE_BYTES_PER_ROW
    tb, sb = 2 * (1 + NTILE), 8 * NSP
    rec = state[: T * RECORD_BYTES][: rows * RECORD_BYTES]
    til = state[T * RECORD_BYTES: T * (RECORD_BYTES + tb)][: rows * tb]
    sup = state[T * (RECORD_BYTES + tb):][: rows * sb]
    return torch.cat([rec, til, sup])


class ScoreFunction(torch.autograd.Function):
    """Autograd wrapper of the scoring core:

    ``logprob = ScoreFunction.apply(hidden, weight, target, temperature, top_k, top_p, min_p,
    ignore_index, pre_gemm_temperature, lane)`` (arguments after ``target`` optional, as in
    ``forward``).  The backward recomputes through ``backward`` with the
    incoming gradient as ``grad_logprob``; the weight gradient is returned in
    the weight's dtype."""

    @staticmethod
    def forward(ctx, hidden, weight, target, temperature=None, top_k=None, top_p=None, min_p=None,
                ignore_index=None, pre_gemm_temperature=None, lane="fp32"):
        opts = dict(ignore_index=ignore_index, pre_gemm_temperature=pre_gemm_temperature, lane=lane)
        logprob, state = forward(hidden, weight, target, temperature, top_k, top_p, min_p, **opts)
        ctx.save_for_backward(hidden, weight, target, state)
        ctx.meta = (temperature, top_k, top_p, min_p)
        ctx.opts = opts
        return logprob

    @staticmethod
    def backward(ctx, g):
        hidden, weight, target, state = ctx.saved_tensors
        gh, gw = backward(hidden, weight, target, state, g.float().contiguous(), *ctx.meta,
                          need_hidden=ctx.needs_input_grad[0], need_weight=ctx.needs_input_grad[1], **ctx.opts)
        if gw is not None:
            gw = gw.to(weight.dtype)
        return (gh, gw) + (None,) * 8
