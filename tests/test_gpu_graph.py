"""A training step captured once into a HIP graph and replayed gives the eager step's bits.

The step is the 2-layer MLP of the training tests (256 -> 512 -> 10, ReLU, softmax
cross-entropy, batch 64, static loss scale 1024, SGD lr 0.01 momentum 0.9): "Mixed Precision
Training", long-form analysis page, §3.4 "The Integrated Training Procedure", Steps 1-7. At
this size every kernel runs for microseconds, so the host's launch cost bounds the step; a
graph replays the step's nine launches with one call. Every entry point on the step's path
only launches kernels on the caller's stream (no allocation, no memset, no host
synchronisation), which is what capture needs.

Two copies of the same state: one steps eagerly, the other is captured once and replayed.
Between replays the eager copy runs its step and the host synchronises; after every replay
the masters, momenta, binary16 weights, loss and scaler words of the two copies must be
bitwise equal.
"""
import numpy as np
import pytest
import torch

import mixed_precision_neural_amd as mp
import workloads
from gpu_util import dev_f16, dev_f32, host_bits16, require_gpu

pytestmark = pytest.mark.gpu


class C1State:
    def __init__(self, cfg):
        self.cfg = cfg
        self.S = mp.Scaler(cfg.scale, cfg.dynamic, cfg.growth_interval)
        self.W = [dev_f32(cfg.W1), dev_f32(cfg.W2)]
        self.V = [torch.zeros_like(w) for w in self.W]
        self.W16 = [mp.round_f32_to_f16(w) for w in self.W]
        self.G = [torch.zeros(w.shape, dtype=torch.float16, device="cuda") for w in self.W]
        self.pl = mp.ParamList(self.W, self.V, self.G, self.W16)
        self.X = dev_f16(cfg.X16)
        self.y = torch.from_numpy(cfg.labels).cuda()
        self.Z1 = torch.empty((64, 512), dtype=torch.float16, device="cuda")
        self.H1, self.dZ1 = torch.empty_like(self.Z1), torch.empty_like(self.Z1)
        self.Z2 = torch.empty((64, 10), dtype=torch.float16, device="cuda")
        self.dZ2 = torch.empty_like(self.Z2)
        self.loss = torch.zeros(1, dtype=torch.float32, device="cuda")
        self.ws = torch.empty(mp.loss_softmax_ce_workspace(64, 10), dtype=torch.uint8, device="cuda")

    def step(self):
        """Fused ReLU epilogues, the overflow flag from the weight-gradient epilogues, one
        update pass, the scaler update: the launches only, on the current stream."""
        c = self.cfg
        mp.linear_fwd_act(mp.RELU, self.X, self.W16[0], Z=self.Z1, H=self.H1)
        mp.linear_fwd(self.H1, self.W16[1], Y=self.Z2)
        mp.loss_softmax_ce(self.Z2, self.y, self.S, self.loss, self.dZ2, workspace=self.ws)
        mp.linear_wgrad(self.dZ2, self.H1, dW=self.G[1], found_inf=self.S.found_inf_ptr)
        mp.linear_dgrad_act(mp.RELU, self.dZ2, self.W16[1], self.Z1, dZ=self.dZ1)
        mp.linear_wgrad(self.dZ1, self.X, dW=self.G[0], found_inf=self.S.found_inf_ptr)
        mp.step(self.pl, self.S, c.lr, c.momentum, c.weight_decay, flags=mp.MP_GRADS_PRECHECKED)
        self.S.update()

    def snapshot(self):
        torch.cuda.synchronize()
        return ([w.cpu().numpy().view(np.uint32).copy() for w in self.W + self.V] +
                [host_bits16(h) for h in self.W16] +
                [self.loss.cpu().numpy().view(np.uint32).copy(), self.S.raw()])


def test_c1_step_graph_replays_match_eager_steps():
    require_gpu()
    cfg = workloads.c1()
    eager, graphed = C1State(cfg), C1State(cfg)
    torch.cuda.synchronize()
    # one eager step on both (library and stream warm-up before capture)
    eager.step(); graphed.step()
    assert all(np.array_equal(a, b) for a, b in zip(eager.snapshot(), graphed.snapshot()))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        graphed.step()                     # recorded, not run
    for t in range(6):
        eager.step()
        g.replay()
        a, b = eager.snapshot(), graphed.snapshot()
        names = ["W1", "W2", "V1", "V2", "W16_1", "W16_2", "loss", "scaler"]
        bad = [n for n, x, y in zip(names, a, b) if not np.array_equal(x, y)]
        assert not bad, (t, bad)
    # the run trains and never overflows at this scale
    st = graphed.S.read()
    assert st["skipped_steps"] == 0 and st["scale"] == cfg.scale
    eager.pl.close(); graphed.pl.close()
