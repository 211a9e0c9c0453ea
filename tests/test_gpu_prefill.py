"""The matrix-core prefill kernel against the CPU oracle, through the C ABI
(needs an MI355X).

Every format but the bitmap (whose prefill runs through the decode kernels),
with outliers and rank terms of every factor type, fp16 and bf16 activations,
on shapes with partial 128-row tiles in both M and N and a partial last K step;
skewed outliers and rows holding every column as an outlier (long per-(tile,
step) lists); a clamped layer; bitwise determinism.
"""
import sys

import numpy as np
import pytest

from gpu_util import check_bound, gpu_forward, gpu_layer, to_device_x, torch_cuda
from synth.layers import LogicalLayer, bf16_bits_from_f32, draw_csr_skewed, make_layer, make_x

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


SHAPES = {1: (1210, 300), 2: (1000, 290), 3: (768, 270), 5: (1450, 330)}


@pytest.mark.parametrize("cfg", [1, 2, 3, 5])
def test_prefill_configs(cfg):
    path = "prefill"
    K, N = SHAPES[cfg]
    layer = make_layer(cfg, 1 if cfg == 3 else 0, K=K, N=N)
    mod = gpu_layer(layer, max_M=300)
    for M in (33, 257, 300):
        x = make_x(cfg, 1 if cfg == 3 else 0, M, K=K)
        say(path, layer.name, "M", M)
        check_bound(gpu_forward(layer, x, path=path, mod=mod), layer, x, what=f"{path} {layer.name} M={M}")
    mod.close()


def test_prefill_plain_integer_formats():
    r = np.random.default_rng(31)
    K, N = 700, 270
    for dense, lo, hi in (("int4", -8, 8), ("int8", -127, 128)):
        q = r.integers(lo, hi, size=(N, K)).astype(np.int8)
        s = r.uniform(0.001, 0.01, N).astype(np.float16)
        lay = LogicalLayer(K=K, N=N, dense=dense, qvals=q, row_scale=s)
        x = r.normal(0, 1, (260, K)).astype(np.float16)
        say("prefill plain", dense)
        check_bound(gpu_forward(lay, x, path="prefill"), lay, x, what=dense)
        layb = lay.with_(x_dtype="bf16")
        xb = bf16_bits_from_f32(r.normal(0, 1, (40, K)))
        check_bound(gpu_forward(layb, xb, path="prefill"), layb, xb, what=dense + " bf16")


@pytest.mark.parametrize("cfg", [2, 1])
def test_prefill_outlier_stress(cfg):
    # cfg 2: the 128 x 128 kernel (4-bit LUT); cfg 1: the wide 3-bit LUT kernel.
    # Full rows make per-(tile, K step) lists far longer than one entry per thread.
    r = np.random.default_rng(23)
    K, N = 900, 300
    rp, col, val = draw_csr_skewed(r, r, N, K, density=0.01)
    base = make_layer(cfg, 0, K=K, N=N)
    lay = base.with_(csr_row_ptr=rp, csr_col=col, csr_val=val)
    x = make_x(cfg, 0, 70, K=K)
    say("prefill skewed csr", cfg)
    check_bound(gpu_forward(lay, x, path="prefill"), lay, x, what="skewed csr")
    # rows holding every column as an outlier
    rp2 = np.zeros(N + 1, np.int32); rp2[6:] = K; rp2[200:] = 2 * K
    cols = np.concatenate([np.arange(K), np.arange(K)]).astype(np.int32)
    lay2 = base.with_(csr_row_ptr=rp2, csr_col=cols, csr_val=r.normal(0, 0.2, 2 * K).astype(np.float16))
    check_bound(gpu_forward(lay2, x, path="prefill"), lay2, x, what="full rows csr")
    xb = bf16_bits_from_f32(r.normal(0, 1, (130, K)))
    lay3 = lay2.with_(x_dtype="bf16")
    check_bound(gpu_forward(lay3, xb, path="prefill"), lay3, xb, what="full rows csr bf16")


def test_prefill_rank_and_clamp():
    from test_gpu_parity import _with_lowrank
    for kind, xdt, rank, group in (("int4", "f16", 128, 128), ("bf16", "bf16", 64, 128), ("fp16", "f16", 40, 128)):
        base = make_layer(1, 0, K=1300, N=290).with_(x_dtype=xdt)
        lay = _with_lowrank(base, kind, rank, group, seed=rank)
        rr = np.random.default_rng(rank)
        xf = rr.normal(0, 1, (100, 1300))
        x = bf16_bits_from_f32(xf) if xdt == "bf16" else xf.astype(np.float16)
        say("prefill rank", kind, xdt, rank)
        check_bound(gpu_forward(lay, x, path="prefill"), lay, x, what=f"rank {kind} {xdt}")
    r = np.random.default_rng(4)
    q = r.integers(-127, 128, size=(290, 640)).astype(np.int8)
    clamp = LogicalLayer(K=640, N=290, dense="int8", qvals=q, row_scale=np.full(290, 0.01, np.float16),
                         act_clamp=np.float16(1.5))
    xc = r.normal(0, 2, (65, 640)).astype(np.float16)
    check_bound(gpu_forward(clamp, xc, path="prefill"), clamp, xc, what="clamp")


def test_prefill_deterministic():
    torch = torch_cuda()
    layer = make_layer(5, 0, K=2000, N=300)
    x = make_x(5, 0, 300, K=2000)
    mod = gpu_layer(layer, max_M=300)
    xd = to_device_x(x, layer.x_dtype)
    y1 = mod.forward(xd, path="prefill").cpu().numpy()
    y2 = mod.forward(xd, path="prefill").cpu().numpy()
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))
    check_bound(y1.astype(np.float64), layer, x, what="determinism")
    mod.close()
