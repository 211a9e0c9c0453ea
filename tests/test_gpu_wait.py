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
