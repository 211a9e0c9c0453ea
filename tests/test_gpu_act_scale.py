"""Per-channel activation scaling (SLiM's output-error variant) on the GPU,
against the CPU oracle, through the C ABI (needs an MI355X).

Bit-exact: on an identity layer every output is one scaled activation, so
y must equal the oracle's x'' element by element (clamp, product, rounding
to the activation type).  Floating point: every workload's formats, every
forward path, within 1e-3 * |x'| |W_hat|^T of the fp64 oracle.
"""
import sys

import numpy as np
import pytest

import oracle
from gpu_util import check_bound, gpu_forward, gpu_layer, to_device_x, torch_cuda
from synth.layers import LogicalLayer, bf16_bits_from_f32, make_layer, make_x, with_act_scale

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


SMALL = {1: (1210, 200), 2: (1000, 150), 3: (768, 130), 4: (1280, 140), 5: (1450, 190)}


def _identity_layer(K, x_dtype, clamp, seed, scaled=True):
    # int8 q = I, scale 1: y[m, n] = x''[m, n] for n < K
    q = np.eye(K, dtype=np.int8)
    lay = LogicalLayer(K=K, N=K, dense="int8", qvals=q, row_scale=np.ones(K, np.float16), x_dtype=x_dtype,
                       act_clamp=None if clamp is None else np.float16(clamp))
    return with_act_scale(lay, seed=seed, frac=0.3) if scaled else lay


def _x_rounding(M, K, x_dtype, seed):
    # activations with full significands (so the products need rounding),
    # a spread of exponents, small values near the fp16 subnormals, and signs
    r = np.random.default_rng(seed)
    v = r.choice([-1.0, 1.0], size=(M, K)) * r.uniform(1.0, 2.0, size=(M, K)) * np.exp2(r.integers(-16, 6, (M, K)))
    if x_dtype == "f16":
        return v.astype(np.float16)
    return bf16_bits_from_f32(v.astype(np.float32))


# K = 264: the row-wise kernel (batch 1) and the matrix-core decode kernel edit
# raw activations while staging them; K = 262 (rows not 16-byte aligned) and
# the batch-3 row-wise kernel read them from the prep kernel; so does prefill
@pytest.mark.parametrize("x_dtype", ["f16", "bf16"])
@pytest.mark.parametrize("clamp,scaled", [(None, True), (6.0, True), (6.0, False)])
@pytest.mark.parametrize("path,M,K", [("decode", 1, 264), ("decode", 1, 262), ("decode_valu", 3, 264),
                                      ("decode_mfma", 8, 264), ("decode_mfma", 2, 262), ("prefill", 40, 264)])
def test_scaled_activations_bit_exact(x_dtype, clamp, scaled, path, M, K):
    layer = _identity_layer(K, x_dtype, clamp, seed=1, scaled=scaled)
    x = _x_rounding(M, K, x_dtype, seed=2)
    say("identity", x_dtype, clamp, scaled, path, M, K)
    y = gpu_forward(layer, x, path=path, mod=None)
    xpp = oracle.activations(layer, x)
    assert np.array_equal(y, xpp), f"{int((y != xpp).sum())} activations differ"
    if scaled:  # the scaling changed many of them, and some by a rounding
        raw = oracle.activations(layer.with_(xscale_ch=None, xscale=None), x)
        assert (xpp != raw).sum() > M * len(layer.xscale_ch) // 2


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_scaled_forward_all_paths(cfg):
    K, N = SMALL[cfg]
    li = 1 if cfg in (3, 4) else 0
    for path, M in (("decode", 1), ("decode", 2), ("decode_valu", 3), ("decode_mfma", 5), ("decode", 16),
                    ("prefill", 40)):
        layer = with_act_scale(make_layer(cfg, li, K=K, N=N, M_for_clamp=M), seed=cfg, frac=0.02)
        x = make_x(cfg, li, M, K=K)
        say("scaled", layer.name, path, "M", M)
        y = gpu_forward(layer, x, path=path)
        check_bound(y, layer, x, what=f"{layer.name} {path} M={M}")


@pytest.mark.parametrize("cfg,K,N", [(1, 1216, 200), (5, 1456, 190), (3, 768, 130), (1, 16400, 70)])
def test_scaled_batch1_in_kernel_and_long_rows(cfg, K, N):
    # K a multiple of 8: batch 1 edits in the row-wise kernel (with the fused
    # low-rank prologue for workload 5 and 3); K = 16400 takes more than one
    # staging round, so its activations come from the prep kernel
    li = 1 if cfg == 3 else 0
    layer = with_act_scale(make_layer(cfg, li, K=K, N=N), seed=11, frac=0.02)
    for M in (1, 2):
        x = make_x(cfg, li, M, K=K)
        say("scaled batch", layer.name, "M", M)
        y = gpu_forward(layer, x, path="decode")
        check_bound(y, layer, x, what=f"{layer.name} M={M}")


def test_scaled_layer_full_size_sampled_rows():
    # a LLaMA-70B LUT3 + rank-64 layer at its real shape, 1 % of channels scaled
    torch = torch_cuda()
    layer = with_act_scale(make_layer(5, 0), seed=7)
    mod = gpu_layer(layer, max_M=32)
    rows = np.random.default_rng(3).choice(layer.N, size=48, replace=False)
    for M in (1, 16):
        x = make_x(5, 0, M)
        say("scaled full size", layer.name, "M", M)
        y = mod.forward(to_device_x(x, layer.x_dtype)).cpu().numpy().astype(np.float64)
        torch.cuda.synchronize()
        check_bound(y, layer, x, rows=rows, what=f"full size M={M}")
    mod.close()
