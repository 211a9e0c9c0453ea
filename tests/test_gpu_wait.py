"""The bounded wait for x' L inside a decode launch: a give-up is reported, never silent (needs an MI355X).

A forward of a layer with a low-rank part computes t = x' L_hat in its
launch's first workgroups; the workgroups that add the rank term wait for it
with a bounded poll.  The test makes every such wait give up from the host
(cl_set_wait_limit: t is computed but not published, so each wait runs to its
bound and every kernel ends normally) and checks that the outputs that needed
t are NaN, that the next forward returns CL_EHIP once without launching, and
that forwards after it are correct again.
"""
import sys

import numpy as np
import pytest

import compressed_linear_amd as cla
from gpu_util import check_bound, gpu_layer, to_device_x, torch_cuda
from synth.layers import make_layer, make_x

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


# (workload, M, path, K): the batch-1 row kernel with bf16 and with int4
# factors, the row kernel at batch 2 (fp16), the matrix-core decode kernel at
# batch 4 and 8, the batch-1 streaming kernel with bf16 and with int4 factors
CASES = [(5, 1, "decode_valu", 1280), (3, 1, "decode_valu", 1280), (3, 2, "auto", 1280), (5, 4, "auto", 1280),
         (3, 8, "decode_mfma", 1280), (5, 1, "decode_stream", 2600), (3, 1, "decode_stream", 4160)]


@pytest.mark.parametrize("cfg,M,path,K", CASES)
def test_wait_give_up_is_reported(cfg, M, path, K):
    torch = torch_cuda()
    layer = make_layer(cfg, 0, K=K, N=200)
    x = make_x(cfg, 0, M, K=K)
    say("wait give-up", cfg, M, path)
    mod = gpu_layer(layer, max_M=max(M, 8))
    try:
        xd = to_device_x(x, layer.x_dtype)
        y = mod.forward(xd, path=path)
        torch.cuda.synchronize()
        check_bound(y.cpu().numpy().astype(np.float64), layer, x, what="before")

        mod.set_wait_limit(max_polls=4, withhold=True)  # every wait gives up after four polls
        y = mod.forward(xd, path=path)
        torch.cuda.synchronize()
        yv = y.cpu().numpy()
        assert np.isnan(yv).all(), f"{int((~np.isnan(yv)).sum())} outputs are not NaN after the wait gave up"

        mod.set_wait_limit()  # defaults again
        with pytest.raises(cla.ClError) as e:
            mod.forward(xd, path=path)
        assert e.value.status == -4 and "gave up" in str(e.value)

        y = mod.forward(xd, path=path)  # reported once: this one runs, and is right
        torch.cuda.synchronize()
        check_bound(y.cpu().numpy().astype(np.float64), layer, x, what="after")
    finally:
        mod.close()


# A layer created in memory where an earlier layer of the same shape ran the
# batch-1 streaming kernel: every new layer's first forward has epoch 1, so
# tagged partial sums of t left there by the earlier layer carry the tag the
# new layer's readers wait for, unless cl_create clears them.  Short rows make
# the readers ask for t before the new launch's prologue has written it, so a
# stale value shows (a large activation makes the two layers' t differ by far
# more than the bound).
@pytest.mark.parametrize("cfg,K", [(5, 8200), (3, 4160)])
def test_stream_kernel_tags_cleared_at_create(cfg, K):
    import ctypes
    from synth.layers import bf16_bits_from_f32
    torch = torch_cuda()
    layer = make_layer(cfg, 0, K=K, N=190)
    blob, _ = cla.pack(layer)
    L = cla.lib()
    n = L.cl_device_bytes(blob.ctypes.data, 1)
    buf = torch.empty(n + 256, dtype=torch.uint8, device="cuda")
    base = buf.data_ptr() + ((-buf.data_ptr()) % 256)
    stream = torch.cuda.current_stream().cuda_stream
    x0 = make_x(cfg, 0, 1, K=K)
    x1 = x0.copy()
    big = 3.0e5 if layer.x_dtype == "bf16" else 3.0e4
    x1[0, K // 3] = bf16_bits_from_f32(np.array([big], np.float32))[0] if layer.x_dtype == "bf16" else np.float16(big)
    say("tags cleared at create", cfg, K)
    for trial in range(3):
        for i, x in enumerate((x0, x1)):
            h = ctypes.c_void_p()
            assert L.cl_create(blob.ctypes.data, base, n, 1, stream, ctypes.byref(h)) == 0
            xd = to_device_x(x, layer.x_dtype)
            y = torch.empty((1, layer.N), dtype=torch.float32, device="cuda")
            assert L.cl_forward_path(h, 1, xd.data_ptr(), y.data_ptr(), stream, cla.PATH["decode_stream"]) == 0
            torch.cuda.synchronize()
            assert L.cl_destroy(h) == 0
            check_bound(y.cpu().numpy().astype(np.float64), layer, x, what=f"trial {trial} x{i}")
