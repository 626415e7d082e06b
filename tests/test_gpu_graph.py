"""A whole decode step (acceptance walk, path, fused commit + verify with the
pseudo-values carried) captured in a HIP graph and replayed.

The library allocates, clears and synchronises nothing, so every launch is
capturable; each replay must reproduce the eager step bit for bit, with
ordinary eager work and synchronisations between the replays.
"""
import numpy as np
import pytest
import torch

import gdn_synth as gs
from gpu_util import dev, host, upload

pytestmark = pytest.mark.gpu


def test_decode_step_in_a_graph(gpu_lib):
    print("graph: accept -> path -> commit_verify, batch 4, n 64", flush=True)
    batch = 4
    prev, cur = gs.make_config(2, s=3, batch=batch), gs.make_config(2, s=4, batch=batch)
    rng = np.random.default_rng(4)
    draft, verify = gs.make_accept_tokens(rng, prev.parent, p_match=0.8)
    P, C = upload(prev), upload(cur)
    n, H, d = prev.q.shape[1], prev.q.shape[2], prev.q.shape[3]
    prevt = (P["k"], P["v"], P["alpha"], P["beta"], P["parent"])
    ddraft, dverify = dev(draft), dev(verify)
    f32 = dict(dtype=torch.float32, device="cuda")
    i32 = dict(dtype=torch.int32, device="cuda")

    # the previous tree's pseudo-values on S0: its verify with empty paths
    u_prev = torch.empty((batch, n, H, d), **f32)
    S = P["S0"].clone()
    gpu_lib.commit_verify(S, torch.zeros((batch, 13), **i32), torch.zeros(batch, **i32), prevt,
                          P["q"], P["k"], P["v"], P["alpha"], P["beta"], P["parent"],
                          u_out=u_prev)
    torch.cuda.synchronize()
    assert torch.equal(S, P["S0"])

    S_work = P["S0"].clone()
    out = torch.empty((batch, n, H, d), **f32)
    u_new = torch.empty((batch, n, H, d), **f32)
    path = torch.empty((batch, 13), **i32)
    plen = torch.empty(batch, **i32)
    st = torch.empty(batch, **i32)

    def step():
        acc, _, _ = gpu_lib.accept(P["parent"], ddraft, dverify)
        gpu_lib.path(P["parent"], acc, 13, out=path, path_len=plen)
        gpu_lib.commit_verify(S_work, path, plen, prevt, C["q"], C["k"], C["v"], C["alpha"],
                              C["beta"], C["parent"], out=out, u_prev=u_prev, u_out=u_new,
                              status=st)

    def outputs():
        return [host(t).copy() for t in (out, u_new, S_work, path, plen, st)]

    def reset():
        S_work.copy_(P["S0"])
        out.fill_(float("nan"))
        u_new.fill_(float("nan"))
        path.fill_(-5)
        plen.fill_(-5)
        st.fill_(-7)

    reset()
    step()
    torch.cuda.synchronize()
    ref = outputs()
    assert ref[5].tolist() == [0] * batch and (ref[4] > 0).all()

    # warm up on a side stream, then capture
    reset()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    for rep in range(3):
        reset()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = outputs()
        for name, a, b in zip(("out", "u_out", "S", "path", "path_len", "status"), ref, got):
            assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), (rep, name)
        # eager work of the program's own between replays
        step()
        torch.cuda.synchronize()
        print(f"graph replay {rep}: bitwise equal to the eager step", flush=True)
