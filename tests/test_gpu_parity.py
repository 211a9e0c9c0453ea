"""HIP path vs the CPU oracle, through the C ABI (needs an MI355X).

Bit-exact: the debug dequantisation planes (same unpacking code as the
forward) and outputs on hand-derived dyadic cases.  Floating point: every
output within 1e-3 * |x'| |W_hat|^T of the fp64 oracle.
"""
import sys

import numpy as np
import pytest

import compressed_linear_amd as cla
import oracle
from golden_cases import golden_names, load_golden
from gpu_util import check_bound, gpu_forward, gpu_layer, to_device_x, torch_cuda
from synth.layers import (LogicalLayer, absmax_int4_groups, draw_csr, draw_csr_skewed, draw_mask_2_4,
                          draw_mask_half, make_layer, make_x, bf16_bits_from_f32)

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


# reduced shapes: several tiles and chunks plus ragged tails in both K and N
SMALL = {1: (1210, 200), 2: (1000, 150), 3: (768, 130), 4: (1280, 140), 5: (1450, 190)}
SMALL_M = {1: [1, 3], 2: [1, 2], 3: [1, 8, 16], 4: [16, 5], 5: [1, 4, 16, 32]}


@pytest.mark.parametrize("name", golden_names())
@pytest.mark.parametrize("path", ["decode", "prefill"])
def test_golden_exact(name, path):
    say("golden", name, path)
    layer, x, y_exp, _ = load_golden(name)
    y = gpu_forward(layer, x, path=path)
    assert np.array_equal(y, y_exp), (y, y_exp)


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_debug_planes_bit_exact_small(cfg):
    torch = torch_cuda()
    K, N = SMALL[cfg]
    layer = make_layer(cfg, 0, K=K, N=N)
    say("debug planes", layer.name)
    mod = gpu_layer(layer)
    D16, S16, L32, R32 = mod.debug_dequant()
    torch.cuda.synchronize()
    d, s, l, r = oracle.debug_planes(layer)
    assert np.array_equal(D16.cpu().numpy().view(np.uint16), d.view(np.uint16))
    assert np.array_equal(S16.cpu().numpy().view(np.uint16), s.view(np.uint16))
    if l is not None:
        assert np.array_equal(L32.cpu().numpy(), l) and np.array_equal(R32.cpu().numpy(), r)
    mod.close()


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_forward_small(cfg):
    K, N = SMALL[cfg]
    for M in SMALL_M[cfg]:
        layer = make_layer(cfg, 0, K=K, N=N, M_for_clamp=M)
        x = make_x(cfg, 0, M, K=K)
        say("forward", layer.name, "M", M)
        y = gpu_forward(layer, x)
        check_bound(y, layer, x, what=f"{layer.name} M={M}")


def test_prefill_small_lut3_lr():
    layer = make_layer(5, 1, K=1450, N=190)
    for M in (33, 300):
        x = make_x(5, 1, M, K=1450)
        say("prefill", layer.name, "M", M)
        y = gpu_forward(layer, x, path="prefill")
        check_bound(y, layer, x, what=f"prefill M={M}")


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_prefill_small_all_formats(cfg):
    # the matrix-core path at ragged M, N and K (several tiles and a partial one each way)
    K, N = SMALL[cfg]
    for M in (40, 129):
        layer = make_layer(cfg, 1 if cfg in (3, 4) else 0, K=K, N=N, M_for_clamp=M)
        x = make_x(cfg, 1 if cfg in (3, 4) else 0, M, K=K)
        say("prefill all", layer.name, "M", M)
        y = gpu_forward(layer, x, path="prefill")
        check_bound(y, layer, x, what=f"prefill {layer.name} M={M}")


def _with_lowrank(base, kind, rank, group=128, seed=0):
    r = np.random.default_rng(seed)
    Lf = r.normal(0, 0.01, (base.K, rank))
    Rf = r.normal(0, 0.01, (rank, base.N))
    if kind == "fp16":
        return base.with_(lr="fp16", rank=rank, L=Lf.astype(np.float16), R=Rf.astype(np.float16))
    if kind == "bf16":
        return base.with_(lr="bf16", rank=rank, L=bf16_bits_from_f32(Lf), R=bf16_bits_from_f32(Rf))
    Lq, Ls = absmax_int4_groups(Lf, group)
    Rq, Rs = absmax_int4_groups(Rf, group)
    return base.with_(lr="int4", rank=rank, group=group, L=Lq, R=Rq, L_scale=Ls, R_scale=Rs)


# decode low-rank prologue t = x' L: every factor type against both activation
# types, ranks off the 64-column tile, one K slice and many, odd int4 groups,
# small groups, and activation blocks that leave a partial row tile
LOWRANK_CASES = [
    # (factor, x dtype, rank, group, K, N, Ms)
    ("fp16", "f16", 70, 128, 1300, 90, (1, 2, 3, 5)),
    ("bf16", "bf16", 256, 128, 400, 70, (32, 1)),
    ("fp16", "f16", 64, 128, 9000, 40, (1, 16)),
    ("int4", "f16", 64, 33, 1100, 80, (2, 7)),
    ("int4", "bf16", 128, 128, 1500, 60, (4, 1)),
    ("int4", "f16", 16, 4, 600, 50, (1, 3)),
    ("fp16", "bf16", 32, 128, 700, 50, (3,)),
]


@pytest.mark.parametrize("case", LOWRANK_CASES, ids=lambda c: f"{c[0]}-{c[1]}-r{c[2]}-g{c[3]}-K{c[4]}")
def test_decode_lowrank_prologue(case):
    kind, xdt, rank, group, K, N, Ms = case
    base = make_layer(2, 0, K=K, N=N).with_(x_dtype=xdt)
    lay = _with_lowrank(base, kind, rank, group, seed=rank + K)
    r = np.random.default_rng(K)
    for M in Ms:
        xf = r.normal(0, 1, (M, K))
        x = bf16_bits_from_f32(xf) if xdt == "bf16" else xf.astype(np.float16)
        say("lowrank", case, "M", M)
        check_bound(gpu_forward(lay, x, path="decode"), lay, x, what=f"lowrank {case} M={M}")


# batches 2..4 with long K: activation blocks too large for the row-wise kernel's LDS
# (the tile kernel takes them) next to ones that still fit
BIG_LDS_CASES = [(5, 9000, 70, (4, 3)), (3, 11008, 60, (4,)), (2, 16000, 50, (2,))]


@pytest.mark.parametrize("case", BIG_LDS_CASES, ids=lambda c: f"cfg{c[0]}-K{c[1]}")
def test_rows_large_activation_block(case):
    cfg, K, N, Ms = case
    for M in Ms:
        layer = make_layer(cfg, 0, K=K, N=N, M_for_clamp=M)
        x = make_x(cfg, 0, M, K=K)
        say("big lds", layer.name, "M", M)
        check_bound(gpu_forward(layer, x, path="decode"), layer, x, what=f"big lds {layer.name} M={M}")


# The batch-1 streaming kernel (rows of at least 64 chunks): every workload's
# formats with their rank terms, rows split between wavefronts and a short
# last workgroup (N off the rows per workgroup), activation edits, and a
# workgroup whose outliers overflow its staged entries (read from memory)
STREAM_CASES = [
    # (cfg, K, N, variant)
    (5, 2600, 2600, "base"),       # LUT3 + CSR + bf16 rank 64, bf16 activations
    (3, 4160, 1300, "base"),       # INT4 2:4 + int4 rank 128
    (1, 4096, 700, "base"),        # LUT3 + CSR
    (2, 2088, 3000, "act_scale"),  # LUT4 + CSR, per-channel factors edited while staged
    (2, 2088, 2600, "full_rows"),  # four rows with every column an outlier in one workgroup
    (2, 2600, 1500, "fp16_r70"),   # fp16 rank 70
    (2, 2600, 900, "bf16_r256"),   # bf16 rank 256, bf16 activations
    (2, 2600, 600, "int4_r64_g33"),  # int4 rank 64, odd groups
]


@pytest.mark.parametrize("case", STREAM_CASES, ids=lambda c: f"cfg{c[0]}-K{c[1]}-N{c[2]}-{c[3]}")
def test_stream_kernel(case):
    from synth.layers import with_act_scale
    cfg, K, N, variant = case
    layer = make_layer(cfg, 0, K=K, N=N, M_for_clamp=1)
    r = np.random.default_rng(K + N)
    if variant == "act_scale":
        layer = with_act_scale(layer, seed=4)
    elif variant == "full_rows":
        rp = np.zeros(N + 1, np.int64)
        counts = np.zeros(N, np.int64)
        counts[11:15] = K  # rows 11..14: the second workgroup of 11 rows
        rp[1:] = np.cumsum(counts)
        col = np.tile(np.arange(K), 4).astype(np.int32)
        layer = layer.with_(csr_row_ptr=rp.astype(np.int32), csr_col=col,
                            csr_val=r.normal(0, 0.05, len(col)).astype(np.float16))
    elif variant == "fp16_r70":
        layer = _with_lowrank(layer, "fp16", 70, seed=1)
    elif variant == "bf16_r256":
        layer = _with_lowrank(layer.with_(x_dtype="bf16"), "bf16", 256, seed=2)
    elif variant == "int4_r64_g33":
        layer = _with_lowrank(layer, "int4", 64, group=33, seed=3)
    xf = r.normal(0, 1, (1, K))
    x = bf16_bits_from_f32(xf) if layer.x_dtype == "bf16" else xf.astype(np.float16)
    say("stream", case)
    mod = gpu_layer(layer, max_M=2)
    try:
        ys = gpu_forward(layer, x, path="decode_stream", mod=mod)
        check_bound(ys, layer, x, what=f"stream {case}")
        yr = gpu_forward(layer, x, path="decode_valu", mod=mod)  # the row-wise kernel on the same layer
        y_ref, B = oracle.forward_and_bound(layer, x)
        assert (np.abs(ys - yr) <= 2 * B).all()
    finally:
        mod.close()


def test_deterministic():
    torch = torch_cuda()
    layer = make_layer(5, 0, K=1450, N=190)
    x = make_x(5, 0, 4, K=1450)
    mod = gpu_layer(layer)
    xd = to_device_x(x, layer.x_dtype)
    y1 = mod.forward(xd).cpu().numpy()
    y2 = mod.forward(xd).cpu().numpy()
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))
    mod.close()


def test_stress_skewed_csr_and_tiny_shapes():
    r = np.random.default_rng(21)
    K, N = 1000, 257
    rp, col, val = draw_csr_skewed(r, r, N, K, density=0.01)
    base = make_layer(2, 0, K=K, N=N)
    lay = base.with_(csr_row_ptr=rp, csr_col=col, csr_val=val)
    x = make_x(2, 0, 3, K=K)
    say("stress skewed", lay.name)
    check_bound(gpu_forward(lay, x), lay, x, what="skewed csr")
    # a row holding every column as an outlier
    rp2 = np.zeros(N + 1, np.int32); rp2[6:] = K
    lay2 = base.with_(csr_row_ptr=rp2, csr_col=np.arange(K, dtype=np.int32),
                      csr_val=r.normal(0, 0.2, K).astype(np.float16))
    check_bound(gpu_forward(lay2, x), lay2, x, what="full row csr")
    # N = 1, K = 2, single activation
    tiny = make_layer(1, 0, K=2, N=1)
    xt = make_x(1, 0, 1, K=2)
    check_bound(gpu_forward(tiny, xt), tiny, xt, what="1x2")
    # odd K (activations restaged with a padded stride)
    odd = make_layer(1, 0, K=333, N=65)
    xo = make_x(1, 0, 2, K=333)
    check_bound(gpu_forward(odd, xo), odd, xo, what="odd K")


def test_plain_integer_formats_and_bf16_activations():
    r = np.random.default_rng(5)
    K, N = 900, 100
    for dense, lo, hi in (("int4", -8, 8), ("int8", -127, 128)):
        q = r.integers(lo, hi, size=(N, K)).astype(np.int8)
        s = r.uniform(0.001, 0.01, N).astype(np.float16)
        lay = LogicalLayer(K=K, N=N, dense=dense, qvals=q, row_scale=s)
        x = r.normal(0, 1, (3, K)).astype(np.float16)
        say("plain", dense)
        check_bound(gpu_forward(lay, x), lay, x, what=dense)
        layb = lay.with_(x_dtype="bf16")
        xb = bf16_bits_from_f32(r.normal(0, 1, (2, K)))
        check_bound(gpu_forward(layb, xb), layb, xb, what=dense + " bf16")
    lay4 = make_layer(2, 0, K=K, N=N).with_(x_dtype="bf16")
    xb = bf16_bits_from_f32(r.normal(0, 1, (5, K)))
    check_bound(gpu_forward(lay4, xb), lay4, xb, what="lut4 bf16")


def test_cross_format_2_4_equals_bitmap():
    r = np.random.default_rng(8)
    K, N = 512, 70
    keep = draw_mask_2_4(r, N, K)
    q = r.integers(-8, 8, size=(N, K)).astype(np.int8)
    s = r.uniform(0.01, 0.02, N).astype(np.float16)
    a = LogicalLayer(K=K, N=N, dense="int4", mask="2:4", qvals=q, keep=keep, row_scale=s)
    b = LogicalLayer(K=K, N=N, dense="int8", mask="bitmap", qvals=q, keep=keep, row_scale=s)
    x = r.normal(0, 1, (4, K)).astype(np.float16)
    ya, yb = gpu_forward(a, x), gpu_forward(b, x)
    check_bound(ya, a, x, what="2:4")
    check_bound(yb, b, x, what="bitmap")
    y_ref, B = oracle.forward_and_bound(a, x)
    assert (np.abs(ya - yb) <= 2 * B).all()


def test_errors_on_device():
    torch = torch_cuda()
    layer = make_layer(1, 0, K=100, N=64)
    mod = gpu_layer(layer, max_M=4)
    x = to_device_x(make_x(1, 0, 5, K=100), "f16")
    with pytest.raises(cla.ClError):
        mod.forward(x)                 # M above max_M
    assert cla.lib().cl_forward(mod._h, 0, x.data_ptr(), x.data_ptr(), None) == -1   # M = 0
    with pytest.raises(ValueError):
        mod.forward(x[:1, :98].contiguous())  # wrong K (caught in the binding)
    mod.close()
