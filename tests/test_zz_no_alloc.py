"""cl_fit_lut_noalloc -- the LUT fitter for callers that cannot allocate -- against cl_fit_lut (needs an MI355X).

Both run the same kernels; the variant's work buffer is the library's static
per-device scratch.  Two calls in a row, the second on a smaller matrix (so a
stale first call's scratch would show), each compared bit for bit with
cl_fit_lut on the same weights: codes, LUTs, CSR row pointers, columns and
values, and the Lloyd iteration count.
"""
import ctypes
import sys

import numpy as np
import pytest

import compressed_linear_amd as cla
from gpu_util import torch_cuda

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def _weights(N, K, seed):
    r = np.random.default_rng(seed)
    w = r.normal(0, 0.02, (N, K))
    w = np.where(r.random((N, K)) < 0.004, r.normal(0, 0.3, (N, K)), w)
    return w.astype(np.float16)


def _noalloc(Wd, bits, n_out, iters):
    torch = torch_cuda()
    N, K = Wd.shape
    dev = Wd.device
    codes = torch.empty((N, K), dtype=torch.uint8, device=dev)
    lut = torch.empty((N, 1 << bits), dtype=torch.float16, device=dev)
    row_ptr = torch.empty(N + 1, dtype=torch.int32, device=dev)
    col = torch.empty(max(n_out, 1), dtype=torch.int32, device=dev)
    val = torch.empty(max(n_out, 1), dtype=torch.float16, device=dev)
    it = ctypes.c_int64(0)
    st = cla.lib().cl_fit_lut_noalloc(Wd.data_ptr(), N, K, bits, n_out, iters, codes.data_ptr(), lut.data_ptr(),
                                      row_ptr.data_ptr(), col.data_ptr(), val.data_ptr(),
                                      torch.cuda.current_stream(dev).cuda_stream, ctypes.byref(it))
    assert st == 0, cla.lib().cl_last_error().decode()
    return (codes, lut, row_ptr, col[:n_out], val[:n_out]), int(it.value)


@pytest.mark.parametrize("bits", [3, 4])
def test_fit_lut_noalloc_matches_fit_lut(bits):
    torch = torch_cuda()
    dev = torch.device("cuda:0")
    for (N, K, seed) in ((1300, 1000, 1), (190, 640, 2)):  # the second call is smaller
        w = _weights(N, K, seed + 10 * bits)
        Wd = torch.from_numpy(w.view(np.int16)).view(torch.float16).to(dev)
        n_out = int(round(0.0045 * N * K))
        say("noalloc fit", bits, N, K, n_out)
        stats = {}
        ref = cla.fit_lut(Wd, bits, n_out, 20, stats)
        got, iters = _noalloc(Wd, bits, n_out, 20)
        torch.cuda.synchronize()
        for name, a, b in zip(("codes", "lut", "row_ptr", "col", "val"), got, ref):
            assert a.shape == b.shape and a.dtype == b.dtype, name
            assert np.array_equal(a.cpu().numpy().view(np.uint8), b.cpu().numpy().view(np.uint8)), name
        assert iters == stats["total_iters"]
