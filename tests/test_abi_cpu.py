"""Host-side checks of the C ABI: the library loads without a GPU, exports
every function include/stce.h declares, and rejects bad arguments before
anything is launched (no device call is made by these tests)."""
import ctypes
import os
import re

import pytest

from sampling_transform_logprob_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "stce.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(stce_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.LIB_PATH):
        pytest.skip("libstce.so not built")
    return binding.load()


def test_library_exports_every_declared_function(lib):
    names = _declared()
    assert "stce_forward" in names and "stce_backward" in names
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(binding.SYMBOLS)


def test_struct_layouts_match_header(tmp_path):
    assert ctypes.sizeof(binding.Problem) == 128
    assert ctypes.sizeof(binding.RowInfo) == binding.RECORD_BYTES
    assert binding.STATE_BYTES_PER_ROW == binding.RECORD_BYTES + 2 * (1 + binding.NTILE) + 8 * binding.NSP
    # the binding's field offsets against the C compiler's for the header
    fields = [f for f, _ in binding.Problem._fields_]
    src = tmp_path / "layout.c"
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "stce.h"\nint main(void) {\n'
                   '  printf("%zu\\n", sizeof(stce_problem));\n'
                   + "".join(f'  printf("%zu\\n", offsetof(stce_problem, {f}));\n' for f in fields)
                   + "  return 0;\n}\n")
    exe = tmp_path / "layout"
    import subprocess
    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    out = [int(x) for x in subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split()]
    assert out[0] == ctypes.sizeof(binding.Problem)
    assert out[1:] == [getattr(binding.Problem, f).offset for f in fields]


def _prob(**kw):
    d = dict(T=8, H=64, V=100, dtype=binding.DT_BF16)
    d.update(kw)
    p = binding.Problem()
    for k, v in d.items():
        setattr(p, k, v)
    return p


def test_workspace_sizes_are_host_computable(lib):
    f, b = binding.workspace_bytes(_prob())
    assert f > 8 * 100 * 4 and b > 0
    f2, _ = binding.workspace_bytes(_prob(T=100000, chunk_rows=512))
    # bounded by two chunk buffers (keys, tile partials, target keys; the
    # selection of one chunk overlaps the projection of the next) plus the
    # per-row flags: nothing scales with T x V
    assert f2 < 2 * (512 * 101 * 4 + 512 * 16 + 512 * 4) + 100000 * 4 + 4096
    assert lib.stce_state_bytes(10) == 11200


def _last_wave_idle(V, n):
    """Idle fraction of the last wave of one workgroup per compute unit over
    ceil(V / 256) x n output tiles (256 compute units)."""
    tiles = -(-V // 256) * n
    return (-(-tiles // 256) * 256 - tiles) / 256


def test_default_chunking(lib):
    """Default rows per forward chunk (stce_schedule): one chunk up to 4,096
    rows; else two chunks of about T / 2 rows, a multiple of 256 at most two
    token tiles above the half, with the least idle compute over the two
    launches' last waves; more chunks once two buffers of fp32 keys
    (4 C round_up(V, 4) bytes each) would exceed 12 GB; the fp8 lane keeps
    256 n rows, n in 12 .. 16 filling whole waves best (3,840 at
    V = 151,936).  The forward workspace holds the two key buffers."""
    for T in (1, 300, 4096):
        assert binding.schedule(_prob(T=T, H=512, V=151936))[0] == T
    T, V = 16384, 151936
    C = binding.schedule(_prob(T=T, H=5120, V=V))[0]
    nt, half = T // 256, T // 512
    assert C % 256 == 0 and half * 256 <= C <= (half + 2) * 256 and C < T
    waste = {n: _last_wave_idle(V, n) + _last_wave_idle(V, nt - n) for n in range(half, half + 3)}
    assert waste[C // 256] == min(waste.values())
    assert C == 8448                                                   # 33 + 31 token tiles
    ld = -(-V // 4) * 4
    assert binding.workspace_bytes(_prob(T=T, H=5120, V=V))[0] >= 2 * 4 * C * ld
    fp8 = _prob(T=T, H=5120, V=V, dtype=binding.DT_FP8, weight_scale=16)
    assert binding.schedule(fp8)[0] == 3840
    # tie-stress shape: two 16,384-row buffers of keys would be 16.9 GB
    T, V = 32768, 129280
    C = binding.schedule(_prob(T=T, H=7168, V=V))[0]
    assert -(-T // C) >= 3 and 2 * 4 * C * (-(-V // 4) * 4) <= 12e9 and C % 256 == 0
    # an explicit chunk is kept
    assert binding.schedule(_prob(T=T, H=7168, V=V, chunk_rows=4096))[0] == 4096


def test_unsupported_dtype_is_one_actionable_error(lib):
    with pytest.raises(binding.StceError, match="UNSUPPORTED.*dtype 7.*STCE_DT_FP8"):
        binding.workspace_bytes(_prob(dtype=7))


def test_fp8_lane_host_checks(lib):
    """The fp8 lane: H a multiple of 16, weight_scale required, neither the
    bf16 value lane nor the pre-GEMM temperature; its workspaces add the
    quantized hidden rows (codes and scales), and its fused step takes the
    path with row classes (one workspace size)."""
    fp8 = binding.DT_FP8
    with pytest.raises(binding.StceError, match="H=72.*multiple of 16"):
        binding.workspace_bytes(_prob(dtype=fp8, H=72))
    with pytest.raises(binding.StceError, match="UNSUPPORTED.*bf16 value lane"):
        binding.workspace_bytes(_prob(dtype=fp8, flags=binding.PROBLEM_BF16_LANE))
    with pytest.raises(binding.StceError, match="UNSUPPORTED.*pre-GEMM"):
        binding.workspace_bytes(_prob(dtype=fp8, flags=binding.PROBLEM_PRE_GEMM_TEMPERATURE,
                                      pre_gemm_temperature=0.5))
    full, least = binding.fused_workspace_bytes(_prob(dtype=fp8))
    assert full == least > 0
    p = _prob(dtype=fp8)
    p.hidden, p.weight, p.target = 16, 16, 16          # fake, never dereferenced
    st = lib.stce_forward(ctypes.byref(p), ctypes.c_void_p(16), ctypes.c_void_p(16), None, None, 0, None)
    assert st == 1 and b"weight_scale" in lib.stce_last_error()
    T, H, V = 1000, 128, 5000
    f8, b8 = binding.workspace_bytes(_prob(T=T, H=H, V=V, dtype=fp8))
    f16, b16 = binding.workspace_bytes(_prob(T=T, H=H, V=V, dtype=binding.DT_BF16))
    up = lambda x: -(-x // 256) * 256  # noqa: E731
    # forward: codes and scales of one chunk buffer (one chunk here); the
    # rows to re-project are gathered as codes (1 byte, not 2)
    assert f8 - f16 == up(T * H) + up(4 * T) - (up(2 * T * H) - up(T * H))
    # backward: the permuted codes and the per-row scales
    assert b8 - b16 == up(T * H) + up(4 * T)
    for R, H_, msg in ((-1, 64, b"R=-1"), (4, 24, b"H=24")):
        assert lib.stce_fp8_quantize_rows(ctypes.c_void_p(16), R, H_, ctypes.c_void_p(16), ctypes.c_void_p(16),
                                          None) == 1
        assert msg in lib.stce_last_error()
    assert lib.stce_fp8_quantize_rows(None, 0, 64, None, None, None) == 0
    st = lib.stce_fp8_quantize_rows(ctypes.c_void_p(16), 4, 64, ctypes.c_void_p(24), ctypes.c_void_p(16), None)
    assert st == 1 and b"aligned" in lib.stce_last_error()


@pytest.mark.parametrize("kw,msg", [
    (dict(T=0), "T=0"), (dict(H=12), "H=12"), (dict(V=0), "V=0"), (dict(flags=16), "flags"),
    (dict(flags=1, ignore_index=5), "ignore_index=5"),
    (dict(chunk_rows=-1), "chunk_rows"),
    # 512 * round_up(T, 64) bytes must fit a 32-bit buffer record count
    (dict(T=(1 << 22) - 63), "T=4194241"),
])
def test_bad_shapes_are_rejected(lib, kw, msg):
    with pytest.raises(binding.StceError, match=msg):
        binding.workspace_bytes(_prob(**kw))


def test_recompute_all_flag_is_accepted_and_changes_no_size(lib):
    """The flag that makes the backward recompute every row changes neither
    workspace (the recompute's buffers exist for every problem)."""
    base = binding.workspace_bytes(_prob(T=1000, H=64, V=5000))
    assert binding.workspace_bytes(_prob(T=1000, H=64, V=5000, flags=binding.PROBLEM_RECOMPUTE_ALL)) == base


def test_largest_row_count_is_accepted(lib):
    f, b = binding.workspace_bytes(_prob(T=(1 << 22) - 64))
    assert f > 0 and b > 0


@pytest.mark.parametrize("ts", [0.0, -0.5, float("nan"), float("inf")])
def test_bad_pre_gemm_temperature_is_rejected(lib, ts):
    with pytest.raises(binding.StceError, match="pre_gemm_temperature"):
        binding.workspace_bytes(_prob(flags=binding.PROBLEM_PRE_GEMM_TEMPERATURE, pre_gemm_temperature=ts))


def test_pre_gemm_temperature_workspaces_hold_the_scaled_hidden(lib):
    """The scalar pre-GEMM convention keeps h / Ts (operand dtype, T x H) in
    every workspace; nothing else changes."""
    for dt, es in ((binding.DT_BF16, 2), (binding.DT_F32, 4)):
        base = _prob(T=1000, H=136, V=5000, dtype=dt)
        pre = _prob(T=1000, H=136, V=5000, dtype=dt, flags=binding.PROBLEM_PRE_GEMM_TEMPERATURE,
                    pre_gemm_temperature=0.7)
        hs = -(-1000 * 136 * es // 256) * 256
        f0, b0 = binding.workspace_bytes(base)
        f1, b1 = binding.workspace_bytes(pre)
        assert (f1 - f0, b1 - b0) == (hs, hs)
        assert binding.fused_workspace_bytes(pre)[0] - binding.fused_workspace_bytes(base)[0] == hs
        assert binding.schedule(pre) == binding.schedule(base)


def test_bf16_lane_takes_bf16_operands_only(lib):
    with pytest.raises(binding.StceError, match="UNSUPPORTED.*bf16 value lane"):
        binding.workspace_bytes(_prob(dtype=binding.DT_F32, flags=binding.PROBLEM_BF16_LANE))
    lane = _prob(flags=binding.PROBLEM_BF16_LANE | binding.PROBLEM_PRE_GEMM_TEMPERATURE, pre_gemm_temperature=0.5)
    assert binding.workspace_bytes(lane)[0] > 0
    with pytest.raises(ValueError, match="lane"):
        binding.make_problem(None, None, None, lane="fp16")


def test_pre_gemm_temperature_excludes_the_per_row_array(lib):
    p = _prob(flags=binding.PROBLEM_PRE_GEMM_TEMPERATURE, pre_gemm_temperature=0.7)
    p.hidden, p.weight, p.target, p.temperature = 16, 16, 16, 16    # fake, never dereferenced
    st = lib.stce_forward(ctypes.byref(p), ctypes.c_void_p(16), ctypes.c_void_p(16), None, None, 0, None)
    assert st == 1 and b"do not combine" in lib.stce_last_error()
    torch = pytest.importorskip("torch")
    with pytest.raises(ValueError, match="not both"):
        binding.make_problem(torch.zeros(2, 8), torch.zeros(3, 8), torch.zeros(2, dtype=torch.int64),
                             torch.ones(2), pre_gemm_temperature=0.7)


def test_noalloc_forward_rejects_what_its_scratch_cannot_hold(lib):
    """stce_forward_noalloc keeps its workspace in a 64 MiB static array;
    a vocabulary whose single-row chunk needs more is rejected before any
    device call (the pointers here are never dereferenced)."""
    assert lib.stce_noalloc_scratch_bytes() == 64 << 20
    p = _prob(T=4, H=64, V=20_000_000)
    p.hidden, p.weight, p.target = 16, 16, 16
    st = lib.stce_forward_noalloc(ctypes.byref(p), ctypes.c_void_p(16), ctypes.c_void_p(16), None, None)
    assert st == 3 and b"static scratch" in lib.stce_last_error()


def test_forward_rejects_null_and_small_workspace_before_launch(lib):
    p = _prob()
    st = lib.stce_forward(ctypes.byref(p), None, None, None, None, 0, None)
    assert st == 1 and b"required" in lib.stce_last_error()
    p.hidden, p.weight, p.target = 16, 16, 16          # fake, never dereferenced: checks stop first
    st = lib.stce_forward(ctypes.byref(p), ctypes.c_void_p(16), ctypes.c_void_p(16), None, None, 0, None)
    assert st == 3 and b"workspace" in lib.stce_last_error()
    p.hidden = 18
    st = lib.stce_forward(ctypes.byref(p), ctypes.c_void_p(16), ctypes.c_void_p(16), None, None, 0, None)
    assert st == 1 and b"aligned" in lib.stce_last_error()


def test_support_entry_rejects_bad_layout(lib):
    st = lib.stce_support_from_logits(ctypes.c_void_p(16), 2, 10, None, None, None, ctypes.c_void_p(16),
                                      ctypes.c_void_p(16), ctypes.c_void_p(16), None, None, 0, None)
    assert st == 1 and b"multiple of 4" in lib.stce_last_error()


def test_binding_rejects_over_length_metadata():
    torch = pytest.importorskip("torch")
    t = torch.zeros(5)
    with pytest.raises(ValueError, match=r"shape \[4\]"):
        binding._meta("top_p", t, 4, torch.float32, t.device)


def test_decode_state_roundtrip(lib):
    import numpy as np
    raw = np.zeros(3, dtype=np.dtype([("key_thr", "<u4"), ("id_thr", "<i4"), ("n", "<i4"), ("flags", "<u4"),
                                      ("lse", "<f4"), ("lsef", "<f4"), ("m", "<f4"), ("sy", "<f4")]))
    raw["id_thr"] = [5, 6, 7]
    raw["n"] = [1, 2, 3]
    raw["flags"] = [0, 0, 32]
    tiles = np.zeros((3, 32), np.uint16)
    tiles[1, :3] = [2, 9, 4000]                      # row 1 lists tiles 9 and 4000
    sup = np.zeros((3, 128), np.dtype([("id", "<i4"), ("key", "<f4")]))
    sup[2, :2] = [(17, 2.5), (3, -1.25)]             # row 2 lists its support {17, 3}
    torch = pytest.importorskip("torch")
    d = binding.decode_state(torch.from_numpy(np.concatenate([raw.view(np.uint8), tiles.view(np.uint8).ravel(),
                                                              sup.view(np.uint8).ravel()])))
    assert list(d["id_thr"]) == [5, 6, 7] and list(d["n"]) == [1, 2, 3]
    assert list(d["ntile"]) == [0, 2, 0] and list(d["tiles"][1, :2]) == [9, 4000]
    assert list(d["flags"] & binding.FLAG_LISTED) == [0, 0, 32]
    assert list(d["support_ids"][2, :3]) == [17, 3, 0] and list(d["support_keys"][2, :2]) == [2.5, -1.25]


def test_policy_loss_rejects_bad_parameters_before_launch(lib):
    fake = ctypes.c_void_p(16)
    good = dict(objective=1, eps_low=0.2, eps_high=0.28, scale=1.0, advantages=16, old_logprob=16)

    def call(T=4, **kw):
        d = dict(good)
        d.update(kw)
        pg = binding.PgParams(**d)
        return lib.stce_policy_loss(ctypes.byref(pg), T, fake, fake, fake, None, None)

    for kw, msg in ((dict(objective=3), b"objective"), (dict(eps_low=1.0), b"eps_low"),
                    (dict(eps_low=-0.1), b"eps_low"), (dict(eps_high=-1.0), b"eps_high"),
                    (dict(eps_high=float("inf")), b"eps_high"), (dict(scale=float("nan")), b"scale"),
                    (dict(advantages=None), b"required"), (dict(old_logprob=18), b"aligned")):
        assert call(**kw) == 1, kw
        assert msg in lib.stce_last_error(), (kw, lib.stce_last_error())
    assert call(T=0) == 1 and b"T=0" in lib.stce_last_error()
    assert lib.stce_policy_loss(None, 4, fake, fake, fake, None, None) == 1
    assert ctypes.sizeof(binding.PgParams) == 40


def test_fused_workspace_is_host_computable_and_chunk_bounded(lib):
    n, nmin = binding.fused_workspace_bytes(_prob(T=100000, chunk_rows=512))
    V, Vp, H = 100, 128, 64
    # one chunk's keys, partials, target keys, row gradients and token-major
    # dz; the vocab-major dz of a group of chunks (at most the 8 GB slice
    # budget, here all rows); the transposed weight and hidden, the split
    # partials and the row flags
    per_chunk = 2 * 512 * (104 * 4 + 16 + 4) + 512 * 4 + 2 * 512 * Vp
    groups = 2 * Vp * 100352
    assert n < per_chunk + groups + 2 * H * Vp + 2 * H * 100032 + 16 * 4 * 512 * H + 100000 * 4 + 16 * 4096
    big = _prob(T=16384, H=5120, V=151936)
    nb, _ = binding.fused_workspace_bytes(big)
    assert 11.8e9 < nb < 12.1e9    # keys 2 x 2.5 GB, vocab-major dz 5 GB, transposed weight 1.6 GB, ...
    # the minimum keeps one chunk per weight-gradient group
    assert nmin == n - 2 * Vp * 512 * (-(-100000 // 512) - 1)
    n2 = binding.fused_workspace_bytes(_prob(T=100000, chunk_rows=100))[1]   # rounded up to 128 rows
    assert n2 > binding.fused_workspace_bytes(_prob(T=100000, chunk_rows=64))[1]


def test_fused_workspace_of_the_classed_path(lib):
    """A bf16 problem with a filter array (or the fp8 lane) takes the fused
    step's path with row classes: one size (no weight-gradient groups), the
    rows' gradients and then the larger of the forward's and the backward's
    workspaces, which the step uses one after the other."""
    T, H, V = 16384, 5120, 151936
    dense, _ = binding.fused_workspace_bytes(_prob(T=T, H=H, V=V))
    for kw in (dict(top_k=16), dict(top_p=16), dict(min_p=16), dict(top_k=16, dtype=binding.DT_FP8),
               dict(dtype=binding.DT_FP8)):
        full, least = binding.fused_workspace_bytes(_prob(T=T, H=H, V=V, **kw))
        fwd, bwd = binding.workspace_bytes(_prob(T=T, H=H, V=V, **kw))
        assert full == least == 4 * T + max(fwd, bwd), kw
        assert full < dense
    # fp32 operands keep the dense path whatever the filters
    f32, f32min = binding.fused_workspace_bytes(_prob(T=T, H=H, V=V, dtype=binding.DT_F32, top_k=16))
    assert f32 > f32min


def test_fused_step_rejects_bad_arguments_before_launch(lib):
    fake = ctypes.c_void_p(16)
    p = _prob()
    p.hidden, p.weight, p.target = 16, 16, 16       # fake, never dereferenced: checks stop first
    good = dict(objective=1, eps_low=0.2, eps_high=0.28, scale=1.0, advantages=16, old_logprob=16)

    def call(pg_kw=None, state=fake, loss=fake, ws=None, nbytes=0):
        d = dict(good)
        d.update(pg_kw or {})
        pg = binding.PgParams(**d)
        return lib.stce_fused_policy_step(ctypes.byref(p), ctypes.byref(pg), fake, state, loss, None, None, None,
                                          None, 0, None, ws, nbytes, None)

    for kw, msg in ((dict(objective=0), b"objective"), (dict(eps_low=1.5), b"eps_low"),
                    (dict(scale=float("inf")), b"scale"), (dict(advantages=None), b"required")):
        assert call(kw) == 1 and msg in lib.stce_last_error(), kw
    assert call(state=None) == 1 and b"required" in lib.stce_last_error()
    assert call(state=ctypes.c_void_p(20)) == 1 and b"aligned" in lib.stce_last_error()
    assert call() == 3 and b"workspace" in lib.stce_last_error()
    assert lib.stce_fused_policy_step(ctypes.byref(p), None, fake, fake, fake, None, None, None, None, 0, None,
                                      None, 0, None) == 1
    n = ctypes.c_size_t()
    assert lib.stce_fused_workspace_bytes(ctypes.byref(_prob(T=0)), ctypes.byref(n), None) == 1


def test_plain_c_program_links_and_sizes_a_problem(lib, tmp_path):
    """The header is C99 and the library links into a plain C program: the
    program sizes the headline problem's workspaces and reads a host error
    (no device call)."""
    import shutil
    import subprocess
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    src = tmp_path / "abi.c"
    src.write_text(r'''
#include <stdio.h>
#include <string.h>
#include "stce.h"
int main(void) {
  stce_problem p;
  memset(&p, 0, sizeof p);
  p.T = 16384; p.H = 5120; p.V = 151936; p.dtype = STCE_DT_BF16;
  size_t f = 0, b = 0, fu = 0, fm = 0;
  if (stce_workspace_bytes(&p, &f, &b) != STCE_OK) return 1;
  if (stce_fused_workspace_bytes(&p, &fu, &fm) != STCE_OK) return 2;
  p.H = 12;
  stce_status s = stce_workspace_bytes(&p, &f, &b);
  printf("%zu %zu %zu %zu %d %s\n", f, b, fu, fm, (int)s, stce_last_error());
  return s == STCE_E_ARG ? 0 : 3;
}
''')
    exe = tmp_path / "abi"
    libdir = os.path.dirname(binding.LIB_PATH)
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe),
                    binding.LIB_PATH, "-Wl,-rpath," + libdir], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split()
    f, b, fu, fm = (int(x) for x in out[:4])
    pf, pb = binding.workspace_bytes(_prob(T=16384, H=5120, V=151936))
    assert (f, b) == (pf, pb) and fu > fm > 0
    assert out[4] == "1" and "H=12" in " ".join(out[5:])
