"""Every dequantisation route of the forward, bit-exact against the oracle (needs an MI355X).

The debug kernel writes D through the row kernel's tables; the other kernels
turn codes into weights their own way (lane-interleaved single-entry tables,
byte permutes over the row's values held in registers, the bitmap's staged
windows, tables built inside each kernel, weights rounded to the matrix-core
input type).  Each route is checked here through the production kernel
itself: activation rows that are one-hot (x[m, k_m] = 1, every other value 0)
make y[m, n] the route's weight at (n, k_m) plus the outlier there, with no
other rounding, for a layer without a low-rank part.

Expected values, from the oracle's planes D and S (fp64) and the readings of
each route (every rounding nearest-even):
  decode kernels (streaming, row-wise, tile, matrix-core): the weight enters the product
      as fp16 LUT value, or (matrix-core kernel, bf16 activations) that value
      rounded to bf16; integer codes exactly, the row scale applied to the
      fp32 sum (q * s is exact in fp32); the outlier is added in fp32:
      y = fp32(D_op + S).
  prefill: the tile holds the weight in the activation type t (LUT value or
      q * s rounded to t), the outlier rounded to t is added in t:
      y = rnd_t(rnd_t(D) + rnd_t(S)).
Small ragged layers are covered at every k; the workloads' full-size layers
at sampled k (chunk, slice and tail edges, and random positions).
"""
import sys

import numpy as np
import pytest

import oracle
from gpu_util import to_device_x, torch_cuda
from synth.layers import (LogicalLayer, bf16_bits_from_f32, draw_csr, draw_lut_codes, draw_mask_2_4,
                          draw_mask_half, make_layer)

pytestmark = pytest.mark.gpu

ONE = {"f16": np.float16(1.0), "bf16": np.uint16(0x3F80)}


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def _fp32(v):
    return np.asarray(v, dtype=np.float64).astype(np.float32).astype(np.float64)


def _planes_at(layer, ks, block=2048):
    """D[:, ks] and S[:, ks] (fp64, [len(ks), N]) for every row, in row blocks."""
    D = np.zeros((len(ks), layer.N))
    S = np.zeros((len(ks), layer.N))
    for r0 in range(0, layer.N, block):
        rows = np.arange(r0, min(layer.N, r0 + block))
        D[:, rows] = oracle.dense_plane(layer, rows)[:, ks].T
        S[:, rows] = oracle.sparse_plane(layer, rows)[:, ks].T
    return D, S


def expected(layer, ks, route):
    D, S = _planes_at(layer, ks)
    t = layer.x_dtype
    lut = layer.dense.startswith("lut")
    if route == "prefill":
        return oracle.round_to_act(oracle.round_to_act(D, t) + oracle.round_to_act(S, t), t)
    D_op = oracle.round_to_act(D, "bf16") if (route == "mfma" and lut and t == "bf16") else D
    return _fp32(D_op + S)


ROUTES = {  # route -> (path, activation rows per launch)
    "stream": ("decode_stream", 1),  # batch-1 streaming kernel (raw activations edited in it when the layer clamps)
    "rows1": ("decode_valu", 1),   # row kernel, one activation row
    "rows4": ("decode_valu", 4),   # row kernel, four activation rows
    "tile": ("decode_valu", 32),   # tile kernel
    "mfma": ("decode_mfma", 32),   # matrix-core decode
    "prefill": ("prefill", None),  # matrix-core prefill, all sampled k in one launch
}


def run_one_hot(mod, layer, ks, route):
    torch = torch_cuda()
    path, per = ROUTES[route]
    ks = np.asarray(ks)
    per = len(ks) if per is None else per
    outs = []
    for i in range(0, len(ks), per):
        kk = ks[i:i + per]
        x = np.zeros((len(kk), layer.K), dtype=np.uint16 if layer.x_dtype == "bf16" else np.float16)
        x[np.arange(len(kk)), kk] = ONE[layer.x_dtype]
        outs.append(mod.forward(to_device_x(x, layer.x_dtype), path=path))
    torch.cuda.synchronize()
    return torch.cat(outs).cpu().numpy().astype(np.float64)


def check_route(mod, layer, ks, route, what):
    y = run_one_hot(mod, layer, ks, route)
    want = expected(layer, ks, route)
    bad = y != want
    if bad.any():
        i, n = np.argwhere(bad)[0]
        raise AssertionError(f"{what} {route}: {int(bad.sum())} of {bad.size} weights differ; first at "
                             f"k={ks[i]} n={n}: {y[i, n]!r} vs {want[i, n]!r}")
    return int(bad.size)


def small_layer(fmt, x_dtype, K, N=200, seed=0, csr=True):
    r = np.random.default_rng([31, seed, K, N])
    kw = dict(K=K, N=N, x_dtype=x_dtype, name=f"{fmt}/{x_dtype}/{K}x{N}")
    if fmt in ("lut3", "lut4"):
        codes, lut = draw_lut_codes(r, r, N, K, int(fmt[3]))
        kw.update(dense=fmt, codes=codes, lut=lut)
    else:
        dense = "int4" if fmt.startswith("int4") else "int8"
        lo = -8 if dense == "int4" else -127
        q = r.integers(lo, -lo if dense == "int8" else 8, size=(N, K)).astype(np.int8)
        # row scales over a range of exponents, so that q * s rounds in the 16-bit types
        s = (r.uniform(1.0, 2.0, N) * np.exp2(r.integers(-12, -2, N))).astype(np.float16)
        kw.update(dense=dense, qvals=q, row_scale=s)
        if fmt == "int4_24":
            kw.update(mask="2:4", keep=draw_mask_2_4(r, N, K))
        elif fmt == "int8_bm":
            kw.update(mask="bitmap", keep=draw_mask_half(r, N, K))
        if dense == "int8":
            kw["act_clamp"] = np.float16(6.0)  # raw activations edited while staging (1 < 6: unchanged)
    if csr:
        rp, col, val = draw_csr(r, r, N, K, density=0.01)
        kw.update(csr_row_ptr=rp, csr_col=col, csr_val=val)
    return LogicalLayer(**kw)


SPAN = {"lut3": 40, "lut4": 32, "int4": 32, "int8": 16}  # weights per 16-byte code chunk


def _routes_for(layer):
    rs = ["tile", "mfma", "prefill"]
    if layer.mask != "bitmap":  # the bitmap decodes on the tile and matrix-core kernels only
        rs = ["rows1", "rows4"] + rs
        span = 64 if layer.mask == "2:4" else SPAN[layer.dense]
        if -(-layer.K // span) >= 64:  # the streaming kernel takes rows of at least 64 chunks
            rs = ["stream"] + rs
    return rs


FORMATS = ["lut3", "lut4", "int4", "int4_24", "int8", "int8_bm"]


# K = 1208: ragged against every chunk span (40, 32, 64, 16, 128 k) and several
# matrix-core K slices; K = 1204 (not a multiple of 8): activations restaged by
# the prep kernel first.  N = 200: ragged against 64-, 128- and 256-row tiles.
@pytest.mark.parametrize("x_dtype", ["f16", "bf16"])
@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("K", [1208, 1204])
def test_every_route_bit_exact_small(fmt, x_dtype, K):
    from gpu_util import gpu_layer
    layer = small_layer(fmt, x_dtype, K)
    mod = gpu_layer(layer, max_M=K)
    try:
        for route in _routes_for(layer):
            ks = np.arange(K)
            if route in ("stream", "rows1"):  # one launch per k: a sample
                ks = np.unique(np.r_[0, 1, 39, 40, 63, 64, K - 2, K - 1, np.random.default_rng(K).integers(0, K, 24)])
            say(layer.name, route, len(ks))
            check_route(mod, layer, ks, route, layer.name)
    finally:
        mod.close()


# INT4 2:4 without outliers (SLiM's form): the prefill runs it on the sparse-A
# instruction with the stored kept values and positions (no zero expansion);
# the matrix-core decode does so with or without outliers.  K = 1204: 19
# chunks (the last 128-k step holds one); K = 260: 5 chunks; N = 200 leaves a
# partial 128-row tile.
@pytest.mark.parametrize("x_dtype", ["f16", "bf16"])
@pytest.mark.parametrize("K", [1208, 1204, 260])
def test_2_4_sparse_instruction_bit_exact(x_dtype, K):
    from gpu_util import gpu_layer
    layer = small_layer("int4_24", x_dtype, K, seed=1, csr=False)
    mod = gpu_layer(layer, max_M=K)
    try:
        for route in ("mfma", "prefill"):
            say(layer.name, "no outliers", route)
            check_route(mod, layer, np.arange(K), route, layer.name + " no outliers")
    finally:
        mod.close()


# The streaming kernel: rows of 65-66 chunks with a ragged last chunk, 2600
# rows (11 per workgroup: slices of 128 chunks cross two or three row
# boundaries and split rows between wavefronts; the last workgroup is short).
STREAM_K = {"lut3": 2568, "lut4": 2088, "int4": 2088, "int4_24": 4168, "int8": 1048}


@pytest.mark.parametrize("x_dtype", ["f16", "bf16"])
@pytest.mark.parametrize("fmt", [f for f in FORMATS if f != "int8_bm"])
def test_stream_route_bit_exact(fmt, x_dtype):
    from gpu_util import gpu_layer
    K = STREAM_K[fmt]
    layer = small_layer(fmt, x_dtype, K, N=2600)
    mod = gpu_layer(layer, max_M=8)
    try:
        span = 64 if fmt == "int4_24" else SPAN[fmt[:4]]
        ks = np.unique(np.r_[0, 1, span - 1, span, 63 * span, 64 * span - 1, K - 2, K - 1,
                             np.random.default_rng(K).integers(0, K, 12)])
        say(layer.name, "stream", len(ks))
        check_route(mod, layer, ks, "stream", layer.name)
    finally:
        mod.close()


def _sampled_ks(K, n, seed):
    """Chunk, slice and tail edges plus n random positions, sorted."""
    edges = [0, 1, 7, 8, 15, 16, 39, 40, 63, 64, 127, 128, 767, 768, 1023, 1024, K - 2, K - 1]
    r = np.random.default_rng(seed)
    return np.unique(np.r_[[e for e in edges if e < K], r.integers(0, K, n)])


def _spread(ks, n):
    return ks[np.unique(np.linspace(0, len(ks) - 1, n).round().astype(int))]


FULL = [(1, 0), (2, "qkv"), (2, "down"), (3, "up"), (4, "up"), (5, "qkv"), (5, "down")]


@pytest.mark.slow
@pytest.mark.parametrize("cfg,name", FULL, ids=lambda v: str(v))
def test_every_route_bit_exact_full_size_sampled(cfg, name):
    from gpu_util import gpu_layer
    layer = make_layer(cfg, name)
    layer = layer.with_(lr="none", rank=0, L=None, R=None, L_scale=None, R_scale=None)  # the routes' weights alone
    ks = _sampled_ks(layer.K, 64, seed=cfg)
    mod = gpu_layer(layer, max_M=len(ks))
    try:
        for route in _routes_for(layer):
            kk = {"stream": _spread(ks, 8), "rows1": _spread(ks, 8), "rows4": _spread(ks, 16),
                  "tile": _spread(ks, 32)}.get(route, ks)
            say(layer.name, route, len(kk))
            check_route(mod, layer, kk, route, layer.name)
    finally:
        mod.close()
