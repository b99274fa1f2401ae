"""GPU test of the bench's multi-stream schedule: the same steps of the
LLaMA-3-8B MLP workload (gate / up / down, 16384 tokens) run with the four
streams the bench times and on one stream in dependency order must give
bit-identical forward and backward outputs -- the events between the
streams order every producer before its consumers."""

import pytest
import torch

import bench
from spectral_split_quantized_amd import metis

from gpu_helpers import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need an MI355X; none is visible")
    metis.load()
    torch.cuda.set_device(0)


def test_multi_stream_step_equals_single_stream():
    dev = torch.device("cuda", 0)
    steps = 3  # a refresh step, then two cached steps
    inputs = bench.build_inputs(steps, dev)
    multi = bench.MetisMLP(dev, streams=3)
    single = bench.MetisMLP(dev, streams=1)
    for t in range(steps):
        say("schedule step %d" % t)
        multi.step(t, inputs)
        torch.cuda.synchronize()
        single.step(t, inputs)
        torch.cuda.synchronize()
        metis.status_sync()
        for name in multi.out:
            for label, a, b in zip(("Y", "dX", "dW"), multi.out[name], single.out[name]):
                assert torch.equal(a, b), "%s %s differs at step %d" % (name, label, t)
