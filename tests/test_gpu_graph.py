"""The benchmark replays each step from a captured HIP graph.  A captured
step must give, on every replay, exactly what the eager launches give: the
path's kernels are deterministic, so the comparison is bitwise.  Replays are
separated by other eager work and synchronisation, and the outputs are
overwritten before each replay."""
import pytest
import torch

import bench
from convolution_voxelised_point_amd import synth

pytestmark = pytest.mark.gpu


def outputs(name, s):
    """Output tensors of a step, restricted to the rows it defines."""
    if name == "lidar":
        return [s.y]
    if name == "train":
        return [s.y, s.dx, s.dw]
    n_o = int(s.n_out.item())
    return [s.y[:n_o], s.out[:n_o], s.n_out]


@pytest.mark.parametrize("name,scale", [("lidar", 0.1), ("train", 0.04), ("down", 0.05)])
def test_graph_replay_matches_eager(ts, name, scale):
    w = synth.make(name, scale)
    setup = {"lidar": bench.setup_subm, "train": bench.setup_train, "down": bench.setup_down}[name]
    s = setup(ts, w)
    s.run_once()
    ref = [t.clone() for t in outputs(name, s)]
    g = bench.capture(s.fns)
    for _ in range(3):
        a = torch.randn(512, 512, device="cuda")
        (a @ a).sum().item()  # unrelated eager work and a synchronisation
        for t in outputs(name, s):
            t.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for t, r in zip(outputs(name, s), ref):
            assert torch.equal(t, r)
