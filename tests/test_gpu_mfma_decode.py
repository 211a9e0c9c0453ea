"""The matrix-core decode kernel (batch 2..32, weights dequantised in registers)
against the CPU oracle, through the C ABI (needs an MI355X).

Every format (the bitmap through its per-lane kept-byte windows), with and
without outliers and rank terms, fp16 and bf16 activations, at batch sizes across the 8 / 16 / 32 staging variants, on
shapes with a partial 128-row tile and a partial K slice; the golden dyadic
cases exactly; bitwise determinism across the split-K reduction; and the same
cases through the vector-ALU decode kernels (forced), which the automatic
choice no longer takes at these batch sizes.
"""
import sys

import numpy as np
import pytest

import compressed_linear_amd as cla
import oracle
from golden_cases import golden_names, load_golden
from gpu_util import check_bound, gpu_forward, gpu_layer, to_device_x, torch_cuda
from synth.layers import LogicalLayer, bf16_bits_from_f32, draw_csr_skewed, make_layer, make_x

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


# (cfg, K, N): partial 128-row tiles and K not a multiple of the slice
SHAPES = {1: (2410, 200), 2: (3000, 330), 3: (2300, 130), 4: (2560, 170), 5: (2900, 190)}
MS = (1, 2, 5, 8, 9, 16, 17, 32)


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_mfma_decode_configs(cfg):
    K, N = SHAPES[cfg]
    layer = make_layer(cfg, 0, K=K, N=N, M_for_clamp=16)
    mod = gpu_layer(layer, max_M=32)
    for M in MS:
        x = make_x(cfg, 0, M, K=K)
        say("mfma decode", layer.name, "M", M)
        y = gpu_forward(layer, x, path="decode_mfma", mod=mod)
        check_bound(y, layer, x, what=f"mfma {layer.name} M={M}")
    mod.close()


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_valu_decode_forced(cfg):
    K, N = SHAPES[cfg]
    layer = make_layer(cfg, 0, K=K, N=N)
    mod = gpu_layer(layer, max_M=32)
    for M in (5, 16, 32):
        x = make_x(cfg, 0, M, K=K)
        say("valu decode", layer.name, "M", M)
        y = gpu_forward(layer, x, path="decode_valu", mod=mod)
        check_bound(y, layer, x, what=f"valu {layer.name} M={M}")
    mod.close()


@pytest.mark.parametrize("name", golden_names())
def test_mfma_golden_exact(name):
    layer, x, y_exp, _ = load_golden(name)
    say("mfma golden", name)
    mod = gpu_layer(layer, max_M=max(2, x.shape[0]))
    y = gpu_forward(layer, x, path="decode_mfma", mod=mod)
    mod.close()
    assert np.array_equal(y, y_exp), (y, y_exp)


def test_mfma_plain_integer_formats():
    r = np.random.default_rng(15)
    K, N = 1900, 150
    for dense, lo, hi in (("int4", -8, 8), ("int8", -127, 128)):
        q = r.integers(lo, hi, size=(N, K)).astype(np.int8)
        s = r.uniform(0.001, 0.01, N).astype(np.float16)
        lay = LogicalLayer(K=K, N=N, dense=dense, qvals=q, row_scale=s)
        mod = gpu_layer(lay, max_M=32)
        for M in (2, 13, 32):
            x = r.normal(0, 1, (M, K)).astype(np.float16)
            say("mfma plain", dense, "M", M)
            check_bound(gpu_forward(lay, x, path="decode_mfma", mod=mod), lay, x, what=f"{dense} M={M}")
        mod.close()
        layb = lay.with_(x_dtype="bf16")
        xb = bf16_bits_from_f32(r.normal(0, 1, (6, K)))
        modb = gpu_layer(layb, max_M=32)
        check_bound(gpu_forward(layb, xb, path="decode_mfma", mod=modb), layb, xb, what=dense + " bf16")
        modb.close()
    lay4 = make_layer(2, 0, K=K, N=N).with_(x_dtype="bf16")
    xb = bf16_bits_from_f32(r.normal(0, 1, (7, K)))
    check_bound(gpu_forward(lay4, xb, path="decode_mfma"), lay4, xb, what="lut4 bf16")


def test_mfma_lowrank_factor_types():
    from test_gpu_parity import _with_lowrank
    for kind, xdt, rank, group in (("fp16", "f16", 70, 128), ("bf16", "bf16", 256, 128), ("int4", "f16", 128, 128),
                                   ("int4", "bf16", 64, 33), ("fp16", "bf16", 32, 128)):
        base = make_layer(2, 0, K=1300, N=150).with_(x_dtype=xdt)
        lay = _with_lowrank(base, kind, rank, group, seed=rank)
        r = np.random.default_rng(rank)
        mod = gpu_layer(lay, max_M=32)
        for M in (3, 16, 32):
            xf = r.normal(0, 1, (M, 1300))
            x = bf16_bits_from_f32(xf) if xdt == "bf16" else xf.astype(np.float16)
            say("mfma lowrank", kind, xdt, rank, group, "M", M)
            check_bound(gpu_forward(lay, x, path="decode_mfma", mod=mod), lay, x,
                        what=f"lowrank {kind} {xdt} r{rank} M={M}")
        mod.close()


def test_mfma_outlier_stress_and_tiny_shapes():
    r = np.random.default_rng(22)
    K, N = 2100, 257
    rp, col, val = draw_csr_skewed(r, r, N, K, density=0.01)
    base = make_layer(2, 0, K=K, N=N)
    lay = base.with_(csr_row_ptr=rp, csr_col=col, csr_val=val)
    x = make_x(2, 0, 12, K=K)
    say("mfma skewed csr")
    check_bound(gpu_forward(lay, x, path="decode_mfma"), lay, x, what="skewed csr")
    # a row holding every column as an outlier
    rp2 = np.zeros(N + 1, np.int32); rp2[6:] = K
    lay2 = base.with_(csr_row_ptr=rp2, csr_col=np.arange(K, dtype=np.int32),
                      csr_val=r.normal(0, 0.2, K).astype(np.float16))
    check_bound(gpu_forward(lay2, x, path="decode_mfma"), lay2, x, what="full row csr")
    # one row, two columns; odd K (restaged activations)
    tiny = make_layer(1, 0, K=2, N=1)
    xt = make_x(1, 0, 2, K=2)
    check_bound(gpu_forward(tiny, xt, path="decode_mfma"), tiny, xt, what="1x2")
    odd = make_layer(5, 0, K=333, N=65)
    xo = make_x(5, 0, 7, K=333)
    check_bound(gpu_forward(odd, xo, path="decode_mfma"), odd, xo, what="odd K")
    # clamp (int8, no mask)
    q = r.integers(-127, 128, size=(70, 640)).astype(np.int8)
    clamp = LogicalLayer(K=640, N=70, dense="int8", qvals=q, row_scale=np.full(70, 0.01, np.float16),
                         act_clamp=np.float16(1.5))
    xc = (r.normal(0, 2, (9, 640))).astype(np.float16)
    check_bound(gpu_forward(clamp, xc, path="decode_mfma"), clamp, xc, what="clamp")


def test_mfma_deterministic_split_k():
    torch = torch_cuda()
    layer = make_layer(5, 0, K=6000, N=300)
    x = make_x(5, 0, 24, K=6000)
    mod = gpu_layer(layer, max_M=32)
    xd = to_device_x(x, layer.x_dtype)
    y1 = mod.forward(xd, path="decode_mfma").cpu().numpy()
    y2 = mod.forward(xd, path="decode_mfma").cpu().numpy()
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))
    check_bound(y1.astype(np.float64), layer, x, what="split-K")
    mod.close()


def test_bitmap_layer_for_batch_1():
    # a bitmap layer created for batch 1 still decodes on the matrix-core kernel
    K, N = SHAPES[4]
    layer = make_layer(4, 0, K=K, N=N, M_for_clamp=1)
    mod = gpu_layer(layer, max_M=1)
    x = make_x(4, 0, 1, K=K)
    say("bitmap max_M 1")
    check_bound(gpu_forward(layer, x, mod=mod), layer, x, what="bitmap max_M=1 auto")
    check_bound(gpu_forward(layer, x, path="decode_mfma", mod=mod), layer, x, what="bitmap max_M=1 mfma")
    check_bound(gpu_forward(layer, x, path="decode_valu", mod=mod), layer, x, what="bitmap max_M=1 tile kernel")
    mod.close()


def test_mfma_path_errors():
    torch = torch_cuda()
    layer = make_layer(1, 0, K=100, N=64)
    mod = gpu_layer(layer, max_M=1)   # created for batch 1: no matrix-core decode workspace
    x = to_device_x(make_x(1, 0, 1, K=100), "f16")
    with pytest.raises(cla.ClError):
        mod.forward(x, path="decode_mfma")
    mod.close()


def test_mfma_bitmap_layers():
    # unstructured masks of other densities (a chunk with no kept value, one
    # with all 128), a row with no kept value, bitmap rows with outliers and a
    # rank term, bf16 activations
    r = np.random.default_rng(41)
    K, N = 1536, 140
    keep = (r.random((N, K)) < 0.3).astype(np.uint8)
    keep[3, :] = 0
    keep[5, 128:256] = 1
    keep[7, 256:384] = 0
    q = r.integers(-127, 128, size=(N, K)).astype(np.int8)
    s = r.uniform(0.001, 0.01, N).astype(np.float16)
    lay = LogicalLayer(K=K, N=N, dense="int8", mask="bitmap", qvals=q, keep=keep, row_scale=s)
    rp, col, val = draw_csr_skewed(r, r, N, K, density=0.005)
    lay_csr = lay.with_(csr_row_ptr=rp, csr_col=col, csr_val=val)
    from test_gpu_parity import _with_lowrank
    lay_lr = _with_lowrank(lay, "int4", 128, 128, seed=9)
    for L_, what in ((lay, "bitmap 30%"), (lay_csr, "bitmap + csr"), (lay_lr, "bitmap + int4 rank")):
        mod = gpu_layer(L_, max_M=32)
        for M in (1, 6, 16, 32):
            x = r.normal(0, 1, (M, K)).astype(np.float16)
            say("mfma", what, "M", M)
            check_bound(gpu_forward(L_, x, path="decode_mfma", mod=mod), L_, x, what=f"{what} M={M}")
        mod.close()
    layb = lay.with_(x_dtype="bf16")
    xb = bf16_bits_from_f32(r.normal(0, 1, (12, K)))
    check_bound(gpu_forward(layb, xb, path="decode_mfma"), layb, xb, what="bitmap bf16")


def test_mfma_clamp_and_prologue_in_launch():
    # the activation clamp applied while staging (K a multiple of 8) and by the
    # prep kernel (odd K), with and without a rank term whose prologue runs in
    # the same launch (it stages, and clamps, the activations too); repeated
    # forwards with new activations on one layer (a stale t would show), and a
    # bitmap prefill whose 32-row blocks each publish their own epoch
    from test_gpu_parity import _with_lowrank
    r = np.random.default_rng(77)
    cases = []
    for K, xdt, kind in ((1536, "f16", "int4"), (1000, "bf16", "bf16"), (1001, "f16", "fp16"), (1003, "bf16", "int4")):
        N = 150
        q = r.integers(-127, 128, size=(N, K)).astype(np.int8)
        base = LogicalLayer(K=K, N=N, dense="int8", qvals=q, row_scale=r.uniform(0.001, 0.01, N).astype(np.float16),
                            act_clamp=np.float16(1.5), x_dtype=xdt)
        cases.append((f"int8 clamp K{K} {xdt}", base))
        cases.append((f"int8 clamp + {kind} rank K{K} {xdt}", _with_lowrank(base, kind, 96, 128, seed=K)))
    lut = make_layer(2, 0, K=1003, N=130).with_(act_clamp=np.float16(2.0))
    cases.append(("lut4 clamp K1003", lut))
    for what, lay in cases:
        mod = gpu_layer(lay, max_M=32)
        for M in (4, 16, 16, 32):
            xf = r.normal(0, 1, (M, lay.K)) * np.where(r.random(lay.K) < 0.02, 30.0, 1.0)
            x = bf16_bits_from_f32(xf) if lay.x_dtype == "bf16" else xf.astype(np.float16)
            say("mfma", what, "M", M)
            check_bound(gpu_forward(lay, x, path="decode_mfma", mod=mod), lay, x, what=f"{what} M={M}")
        mod.close()
    # bitmap + clamp + int4 rank through the prefill (blocks of 32 rows)
    K, N = 1536, 140
    keep = (r.random((N, K)) < 0.5).astype(np.uint8)
    q = r.integers(-127, 128, size=(N, K)).astype(np.int8)
    bm = LogicalLayer(K=K, N=N, dense="int8", mask="bitmap", qvals=q, keep=keep,
                      row_scale=r.uniform(0.001, 0.01, N).astype(np.float16), act_clamp=np.float16(1.5))
    bm_lr = _with_lowrank(bm, "int4", 128, 128, seed=5)
    mod = gpu_layer(bm_lr, max_M=100)
    for M in (100, 16, 70):
        x = (r.normal(0, 1, (M, K)) * np.where(r.random(K) < 0.01, 30.0, 1.0)).astype(np.float16)
        say("bitmap clamp rank M", M)
        check_bound(gpu_forward(bm_lr, x, mod=mod), bm_lr, x, what=f"bitmap clamp rank M={M}")
    mod.close()


@pytest.mark.parametrize("K", [1456, 8200, 28672])
def test_bf16_batch1_rows_staged_as_fp16(K):
    # bf16 activations at batch 1 are staged as fp16 times a power of two fixed
    # by the row's largest magnitude: rows of any range stay within the bound
    layer = make_layer(5, 0, K=K, N=190)
    x = make_x(5, 0, 1, K=K)
    say("bf16 batch 1", K)
    check_bound(gpu_forward(layer, x, path="decode"), layer, x, what="N(0, 1) row")
    for big in (np.float32(3.0e5), np.float32(1.0e30), np.float32(-3.0e38), np.float32(1.2345e-7),
                np.float32(-7.0e-38)):
        xb = x.copy()
        xb[0, K // 3] = bf16_bits_from_f32(np.array([big], np.float32))[0]
        check_bound(gpu_forward(layer, xb, path="decode"), layer, xb, what=f"one value {big}")
    r = np.random.default_rng(K)
    for lo, hi in ((-60, 60), (-130, -100), (-8, 120)):  # whole rows over wide ranges of exponents
        v = r.choice([-1.0, 1.0], K) * r.uniform(1, 2, K) * np.exp2(r.integers(lo, hi, K))
        xw = bf16_bits_from_f32(v.astype(np.float32))[None, :]
        check_bound(gpu_forward(layer, xw, path="decode"), layer, xw, what=f"exponents {lo}..{hi}")
    xz = np.zeros((1, K), np.uint16)  # zero row: the outputs are the rank term of a zero t, i.e. zero
    assert np.array_equal(gpu_forward(layer, xz, path="decode"), np.zeros((1, layer.N)))
    xn = x.copy()
    xn[0, 7] = 0x7F80  # +inf: every output of the row is NaN
    assert np.isnan(gpu_forward(layer, xn, path="decode")).all()


def test_bf16_batch1_staging_exact_within_range():
    # identity layer (int8 q = I, scale 1), bf16 activations: y[n] = x'[n] exactly for
    # every value within 2^29 of the row's largest magnitude; values further below
    # are off by less than 2^-28 of that magnitude
    K = 1200
    layer = LogicalLayer(K=K, N=K, dense="int8", qvals=np.eye(K, dtype=np.int8), row_scale=np.ones(K, np.float16),
                         x_dtype="bf16")
    r = np.random.default_rng(7)
    v = r.choice([-1.0, 1.0], K) * r.uniform(1, 2, K) * np.exp2(r.integers(-20, 9, K))
    v[3] = 2.0 ** 8 * 1.5  # the row's largest magnitude sits in [2^8, 2^9)
    v[10:20] = r.uniform(1, 2, 10) * np.exp2(r.integers(-60, -25, 10))  # more than 2^29 below it
    x = bf16_bits_from_f32(v.astype(np.float32))[None, :]
    say("bf16 staging exactness")
    y = gpu_forward(layer, x, path="decode")
    xf = oracle.activations(layer, x)
    far = np.zeros(K, bool)
    far[10:20] = True
    assert np.array_equal(y[0, ~far], xf[0, ~far])
    assert (np.abs(y[0, far] - xf[0, far]) < 2.0 ** -28 * 2.0 ** 9).all()
