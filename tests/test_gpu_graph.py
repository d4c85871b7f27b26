"""The decode step (one-token append of every layer that writes, then the
decode of every layer) captured into a HIP graph through torch and replayed:
every replay must give the eager step's outputs bit for bit.  The calls
take caller-owned workspace and launch only kernels on the given stream
(no allocation, no memset node), which is what capture needs.  Between
replays the test runs unrelated eager work and synchronizes, and it clears
the outputs, so a replay that skipped or reordered work would show."""
import pytest
import torch

import bench
import datagen
from tests._gpu_harness import note

pytestmark = pytest.mark.gpu

W = datagen.WORKLOADS

CASES = {
    # dense, hd-64 MFMA decode with split-K partitions and their merge
    "tinyllama_shape": W["tinyllama_cla2"].with_(n_layers=4, batch=4, ctx=1024),
    # DepthGraft map: two-source layers on the dot-product kernel
    "depthgraft_map": W["depthgraft"].with_(n_layers=6, dg_stride=2, batch=2, ctx=517),
    # factorized cache: coefficient + residual appends, absorbed decode, merge
    "factorized": W["factorized_64k"].with_(n_layers=4, batch=2, ctx=1024),
}


@pytest.mark.parametrize("case", list(CASES))
def test_graph_replay_matches_eager_step(case):
    wl = CASES[case]
    note(f"[graph] {case}: {wl.n_layers} layers, batch {wl.batch}, ctx {wl.ctx}")
    rig = bench.DecodeRig(wl)
    cs = torch.cuda.Stream()
    rig.stream = cs
    pt = rig.point(wl.batch, wl.ctx)
    assert pt["n_splits"] > 1      # the merge launch is part of the graph

    def step():
        for l in range(wl.n_layers):
            pt["append"](l)
            pt["decode"](l)

    with torch.cuda.stream(cs):
        step()
        step()
    torch.cuda.synchronize()
    ref = [o.clone() for o in pt["outs"]]
    assert all(bool(torch.isfinite(r).all()) for r in ref)

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cs):
        step()
    torch.cuda.synchronize()

    other = torch.randn(1 << 20, device="cuda")
    for rep in range(3):
        for o in pt["outs"]:
            o.fill_(float("nan"))
        other.mul_(1.0001).add_(0.5)          # unrelated eager work between replays
        torch.cuda.synchronize()
        with torch.cuda.stream(cs):
            g.replay()
        torch.cuda.synchronize()
        for l, (a, b) in enumerate(zip(ref, pt["outs"])):
            assert torch.equal(a, b), f"{case}: replay {rep}, layer {l} differs from the eager step"
        note(f"[graph] {case}: replay {rep} equal")
    # eager again after the replays: same outputs
    with torch.cuda.stream(cs):
        step()
    torch.cuda.synchronize()
    for a, b in zip(ref, pt["outs"]):
        assert torch.equal(a, b)
    del g
    rig.release()
