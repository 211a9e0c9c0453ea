"""The matrix-core prefill kernel against the CPU oracle, through the C ABI
(needs an MI355X).

Every format (the bitmap through a dense int8 copy built when the layer is
created for prefill batches, or through the decode kernels otherwise), with outliers and rank terms of every factor type, fp16 and bf16 activations,
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


@pytest.mark.parametrize("lr", ["none", "int4", "fp16"])
def test_prefill_bitmap_dense_copy(lr):
    # INT8 50 % bitmap + clamp (workload 4's format) on a layer created for
    # prefill batches: the INT8 tile loader over the dense int8 copy; ragged K
    # (not a multiple of the 128-k bitmap chunk or the 64-k step), partial tiles,
    # full-row outliers and a rank term
    from synth.layers import absmax_int4_groups
    r = np.random.default_rng(41)
    K, N = 1000, 290
    base = make_layer(4, 0, K=K, N=N, M_for_clamp=64)
    rp, col, val = draw_csr_skewed(r, r, N, K, density=0.01)
    lay = base.with_(csr_row_ptr=rp, csr_col=col, csr_val=val)
    if lr == "int4":
        Lq, Ls = absmax_int4_groups(r.normal(0, 0.01, (K, 32)), 128)
        Rq, Rs = absmax_int4_groups(r.normal(0, 0.01, (32, N)), 128)
        lay = lay.with_(lr="int4", rank=32, group=128, L=Lq, R=Rq, L_scale=Ls, R_scale=Rs)
    elif lr == "fp16":
        lay = lay.with_(lr="fp16", rank=24, L=r.normal(0, 0.01, (K, 24)).astype(np.float16),
                        R=r.normal(0, 0.01, (24, N)).astype(np.float16))
    mod = gpu_layer(lay, max_M=300)
    for M in (33, 129, 300):
        x = make_x(4, 0, M, K=K)
        say("bitmap prefill", lr, "M", M)
        check_bound(gpu_forward(lay, x, path="prefill", mod=mod), lay, x, what=f"bitmap prefill {lr} M={M}")
        # the same layer's batch-1..32 decode still runs the matrix-core decode kernel
    x = make_x(4, 0, 16, K=K)
    check_bound(gpu_forward(lay, x, path="auto", mod=mod), lay, x, what="bitmap decode, prefill-sized layer")
    mod.close()


def test_prefill_bitmap_golden_exact():
    # the hand-derived INT8 bitmap + clamp case through the dense-copy prefill: exact
    from golden_cases import load_golden
    layer, x, y_exp, _ = load_golden("int8_bitmap_clamp_2x8")
    mod = gpu_layer(layer, max_M=64)
    y = gpu_forward(layer, x, path="prefill", mod=mod)
    mod.close()
    assert np.array_equal(y, y_exp), (y, y_exp)
