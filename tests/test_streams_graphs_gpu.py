"""The library on several streams at once and under HIP graph capture: it
keeps no state between calls and, given a workspace, allocates nothing, so
concurrent calls and graph replays must give the eager results bit for bit.
Every replay is checked, with eager work and synchronisation in between."""
import numpy as np
import pytest
import torch

import long_context_decayed_amd as la
from long_context_decayed_amd.inputs import decay_lambdas, qkv_device, state_device
from gpu_helpers import require_gpu, say

pytestmark = pytest.mark.gpu
LAMS = np.array([0.0, 0.3, 0.9, 0.999, 1.0, 0.5, 0.97, 0.7], dtype=np.float32)


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


def _prefill_inputs(seed, dev, N=3000, d=128):
    q, k, v = qkv_device(2, len(LAMS), N, d, seed=seed, device=dev)
    s0 = state_device(2, len(LAMS), d, seed=seed, device=dev)
    return q, k, v, s0


def test_two_streams_at_once(dev):
    say("prefill, backward and decode on two streams at once vs one stream")
    lam = torch.from_numpy(LAMS).to(dev)
    jobs = [_prefill_inputs(400 + i, dev) for i in range(2)]
    ref = []
    for q, k, v, s0 in jobs:
        kv = torch.empty_like(s0)
        o = la.fwd(q, k, v, lam, kv_in=s0, kv_out=kv, block=64)
        g = la.bwd(q, k, v, lam, o, kv_in=s0, dkv_out=kv, dkv_in=True)
        st = s0.clone()
        od = la.decode_step(q[:, :, 0].contiguous(), k[:, :, 0].contiguous(), v[:, :, 0].contiguous(), lam,
                            kv_in=st, kv_out=st)
        ref.append((o, kv) + tuple(g) + (od, st))
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    got = [None, None]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    for i, ((q, k, v, s0), s) in enumerate(zip(jobs, streams)):
        with torch.cuda.stream(s):
            kv = torch.empty_like(s0)
            o = la.fwd(q, k, v, lam, kv_in=s0, kv_out=kv, block=64)
            g = la.bwd(q, k, v, lam, o, kv_in=s0, dkv_out=kv, dkv_in=True)
            st = s0.clone()
            od = la.decode_step(q[:, :, 0].contiguous(), k[:, :, 0].contiguous(), v[:, :, 0].contiguous(), lam,
                                kv_in=st, kv_out=st)
            got[i] = (o, kv) + tuple(g) + (od, st)
    torch.cuda.synchronize()
    for r, g in zip(ref, got):
        for a, b in zip(r, g):
            assert torch.equal(a, b)


@pytest.mark.parametrize("odt", [torch.bfloat16, torch.float32])
def test_prefill_graph_replays(dev, odt):
    say("prefill captured in a graph with its workspace, replayed 3 times", odt)
    q, k, v, s0 = _prefill_inputs(410, dev)
    B, H, N, d = q.shape
    lam = torch.from_numpy(LAMS).to(dev)
    ws = torch.empty(la.workspace_bytes(B, H, N, d, 64), device=dev, dtype=torch.uint8)
    out = torch.empty((B, H, N, d), device=dev, dtype=odt)
    st = s0.clone()
    # eager: the prefill in place on a copy of the state
    st_e = s0.clone()
    o_e = la.fwd(q, k, v, lam, kv_in=st_e, kv_out=st_e, block=64, out_dtype=odt)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up on the side stream, as capture expects
        la.fwd(q, k, v, lam, kv_in=st, kv_out=st, block=64, out=out, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        la.fwd(q, k, v, lam, kv_in=st, kv_out=st, block=64, out=out, workspace=ws)
    for rep in range(3):
        st.copy_(s0)
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, o_e), "replay %d: output" % rep
        assert torch.equal(st, st_e), "replay %d: state" % rep
        # eager work of the program's own between replays
        la.fwd(k, v, q, lam, block=64)
        torch.cuda.synchronize()


def test_backward_graph_replays(dev):
    say("backward captured in a graph with its workspace, replayed 3 times")
    q, k, v, s0 = _prefill_inputs(420, dev, N=1500)
    B, H, N, d = q.shape
    lam = torch.from_numpy(LAMS).to(dev)
    g = qkv_device(B, H, N, d, seed=421, device=dev)[0]
    dsn = state_device(B, H, d, seed=421, device=dev)
    ref = la.bwd(q, k, v, lam, g, kv_in=s0, dkv_out=dsn, dkv_in=True)
    torch.cuda.synchronize()
    ws = torch.empty(la.lib_bwd_workspace_bytes(B, H, N, d), device=dev, dtype=torch.uint8)
    outs = [torch.empty_like(q) for _ in range(3)] + [torch.empty_like(s0)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())

    def run():
        r = la.bwd(q, k, v, lam, g, kv_in=s0, dkv_out=dsn, dkv_in=outs[3], workspace=ws)
        for dst, src in zip(outs[:3], r[:3]):
            dst.copy_(src)

    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    for rep in range(3):
        for t in outs:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip(outs, ref):
            assert torch.equal(a, b), "replay %d" % rep
        la.fwd(q, k, v, lam, block=64)
        torch.cuda.synchronize()


def test_decode_graph_replays(dev):
    say("decode step captured in a graph (state in place), replayed 3 times")
    B, H, d = 64, 8, 128
    q, k, v = (t[:, :, 0].contiguous() for t in qkv_device(B, H, 1, d, seed=430, device=dev))
    lam = torch.from_numpy(decay_lambdas(H)).to(dev)
    s0 = state_device(B, H, d, seed=430, device=dev)
    st = s0.clone()
    o = torch.empty_like(q)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        la.decode_step(q, k, v, lam, kv_in=st, kv_out=st, out=o)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        la.decode_step(q, k, v, lam, kv_in=st, kv_out=st, out=o)
    st.copy_(s0)
    st_e = s0.clone()
    torch.cuda.synchronize()
    for rep in range(3):
        graph.replay()
        torch.cuda.synchronize()
        o_e = la.decode_step(q, k, v, lam, kv_in=st_e, kv_out=st_e)
        torch.cuda.synchronize()
        assert torch.equal(o, o_e), "replay %d: output" % rep
        assert torch.equal(st, st_e), "replay %d: state" % rep
