"""Stream capture: the library enqueues everything on the caller's stream
(the forward's selections on a side stream joined by event waits, no
allocation, no synchronization, no memset), so a forward + policy loss +
backward sequence can be captured in a HIP graph.  The graph is replayed
several times, with eager work and synchronizations between the replays,
and every replay must give the eager results bit for bit."""
import numpy as np
import pytest
import torch

from gpu_helpers import dev, meta_of, say, targets, to_gpu
from sampling_transform_logprob_amd import binding, workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.load()


def test_captured_step_replays_bitwise():
    T, V = 300, 8192
    w = workloads.make("headline", T=T)
    w["W"] = w["W"][:V]
    y = np.asarray(targets(w), np.int64) % V
    G = to_gpu(w, y)
    meta = meta_of(G)
    prob, keep = binding.make_problem(G["h"], G["W"], G["target"], **meta, chunk_rows=128)   # 3 chunks
    fwd_b, bwd_b = binding.workspace_bytes(prob)
    ws_f = torch.empty(fwd_b, dtype=torch.uint8, device=dev())
    ws_b = torch.empty(bwd_b, dtype=torch.uint8, device=dev())
    lp = torch.empty(T, dtype=torch.float32, device=dev())
    st = torch.empty(T * binding.STATE_BYTES_PER_ROW, dtype=torch.uint8, device=dev())
    loss = torch.empty(T, dtype=torch.float32, device=dev())
    g = torch.empty(T, dtype=torch.float32, device=dev())
    gh = torch.empty(T, w["H"], dtype=torch.bfloat16, device=dev())
    gw = torch.empty(V, w["H"], dtype=torch.float32, device=dev())
    rng = np.random.Generator(np.random.PCG64(5))
    adv = torch.from_numpy(rng.standard_normal(T).astype(np.float32)).to(dev())
    old = torch.from_numpy((-rng.exponential(1.0, T)).astype(np.float32)).to(dev())
    pg = binding.PgParams(binding.PG_OBJECTIVES["cispo"], 0.2, 0.28, 1.0 / T, adv.data_ptr(), old.data_ptr(), None)
    L = binding.load()
    import ctypes
    P = ctypes.byref(prob)
    vp = ctypes.c_void_p

    def step(stream):
        s = vp(stream.cuda_stream)
        binding._check(L.stce_forward(P, vp(lp.data_ptr()), vp(st.data_ptr()), None, vp(ws_f.data_ptr()), fwd_b, s))
        binding._check(L.stce_policy_loss(ctypes.byref(pg), T, vp(lp.data_ptr()), vp(loss.data_ptr()),
                                          vp(g.data_ptr()), None, s))
        binding._check(L.stce_backward(P, vp(g.data_ptr()), vp(st.data_ptr()), vp(gh.data_ptr()), vp(gw.data_ptr()),
                                       0, None, vp(ws_b.data_ptr()), bwd_b, s))

    say(f"graph capture: headline T={T} V={V}, 3 chunks")
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        step(side)                     # eager warmup (creates the library's side stream and events)
    torch.cuda.synchronize()
    ref = [t.clone() for t in (lp, st, loss, g, gh, gw)]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        step(side)
    torch.cuda.synchronize()
    for r in range(3):
        for t in (lp, st, loss, g, gh, gw):
            t.zero_()                  # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(("logprob", "state", "loss", "grad", "grad_hidden", "grad_weight"),
                              (lp, st, loss, g, gh, gw), ref):
            ab = a.view(torch.int32) if a.dtype == torch.float32 else a
            bb = b.view(torch.int32) if b.dtype == torch.float32 else b
            assert torch.equal(ab, bb), (r, name)
        say(f"  replay {r}: bitwise equal to the eager step")


def test_captured_fused_step_replays_bitwise():
    T, V = 300, 6000
    w = workloads.make("top_p", T=T)
    w["W"] = w["W"][:V]
    y = np.asarray(targets(w), np.int64) % V
    G = to_gpu(w, y)
    meta = meta_of(G)
    rng = np.random.Generator(np.random.PCG64(6))
    adv = torch.from_numpy(rng.standard_normal(T).astype(np.float32)).to(dev())
    old = torch.from_numpy((-rng.exponential(1.0, T)).astype(np.float32)).to(dev())
    prob, keep = binding.make_problem(G["h"], G["W"], G["target"], **meta, chunk_rows=128)   # 3 chunks
    nb, _ = binding.fused_workspace_bytes(prob)
    ws = torch.empty(nb, dtype=torch.uint8, device=dev())
    out = {k: torch.empty(T, dtype=torch.float32, device=dev()) for k in ("logprob", "loss", "ratio")}
    out["state"] = torch.empty(T * binding.STATE_BYTES_PER_ROW, dtype=torch.uint8, device=dev())
    out["grad_hidden"] = torch.empty(T, w["H"], dtype=torch.bfloat16, device=dev())
    out["grad_weight"] = torch.empty(V, w["H"], dtype=torch.float32, device=dev())
    pg = binding.PgParams(binding.PG_OBJECTIVES["clip"], 0.2, 0.28, 1.0 / T, adv.data_ptr(), old.data_ptr(), None)
    L = binding.load()
    import ctypes
    vp = ctypes.c_void_p

    def step(stream):
        binding._check(L.stce_fused_policy_step(
            ctypes.byref(prob), ctypes.byref(pg), vp(out["logprob"].data_ptr()), vp(out["state"].data_ptr()),
            vp(out["loss"].data_ptr()), vp(out["ratio"].data_ptr()), None, vp(out["grad_hidden"].data_ptr()),
            vp(out["grad_weight"].data_ptr()), 0, None, vp(ws.data_ptr()), nb, vp(stream.cuda_stream)))

    say(f"graph capture, fused step: top_p T={T} V={V}, 3 chunks")
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        step(side)
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in out.items()}
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        step(side)
    torch.cuda.synchronize()
    for r in range(3):
        for v in out.values():
            v.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k, v in out.items():
            a = v.view(torch.int32) if v.dtype == torch.float32 else v
            b = ref[k].view(torch.int32) if ref[k].dtype == torch.float32 else ref[k]
            assert torch.equal(a, b), (r, k)
        say(f"  replay {r}: bitwise equal to the eager step")
