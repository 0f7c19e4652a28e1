"""mp_loss_mse_noalloc through the C-ABI against mp_loss_mse on the same inputs: the loss and the
gradient bit for bit, on two calls in a row, the second with a smaller input (the scratch array
keeps the first call's partials, which the second must not read)."""
import ctypes as C

import numpy as np
import pytest
import torch

import mixed_precision_neural_amd as mp
from gpu_util import dev_f16, host_bits16, host_f32, require_gpu

pytestmark = pytest.mark.gpu


def call_noalloc(y, t, c, sc, loss, dy):
    M, N = y.shape
    st = mp.lib().mp_loss_mse_noalloc(C.c_void_p(y.data_ptr()), C.c_void_p(t.data_ptr()), M, N, C.c_float(c),
                                      sc.ptr, C.c_void_p(loss.data_ptr()), C.c_void_p(dy.data_ptr()),
                                      C.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, st


@pytest.mark.parametrize("shapes", [((2048, 2048), (37, 53)), ((4096, 4096), (1024, 1536))])
def test_noalloc_loss_matches_the_workspace_loss(shapes):
    require_gpu()
    rng = np.random.Generator(np.random.PCG64(17))
    sc = mp.Scaler(2.0 ** 16, True)
    for (M, N), c in zip(shapes, (1058.37, 3.5)):
        y = dev_f16(rng.standard_normal((M, N)).astype(np.float16).view(np.uint16))
        t = dev_f16(rng.standard_normal((M, N)).astype(np.float16).view(np.uint16))
        loss_ref, dy_ref = mp.loss_mse(y, t, c, sc)
        loss = torch.full((1,), -1.0, device="cuda")
        dy = torch.empty((M, N), dtype=torch.float16, device="cuda")
        call_noalloc(y, t, c, sc, loss, dy)
        torch.cuda.synchronize()
        assert host_f32(loss).view(np.uint32)[0] == host_f32(loss_ref).view(np.uint32)[0], (M, N)
        assert np.array_equal(host_bits16(dy), host_bits16(dy_ref)), (M, N)


def test_noalloc_validation_and_empty():
    require_gpu()
    L = mp.lib()
    P = C.c_void_p(0x1000)
    assert L.mp_loss_mse_noalloc(P, P, -1, 8, C.c_float(1.0), P, P, P, None) == 1
    assert L.mp_loss_mse_noalloc(P, P, 8, 8, C.c_float(1.0), None, P, P, None) == 1
    assert L.mp_loss_mse_noalloc(None, None, 0, 8, C.c_float(1.0), P, P, None, None) == 0
