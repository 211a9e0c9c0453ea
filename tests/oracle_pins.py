"""Pins of the CPU oracle against facts that do not come from the oracle.

Each pin takes the oracle module `O` as an argument so that the mutation
tests can run the same pins against deliberately broken copies of it.
The pins use, in turn:
  * hand-derived worked examples (tests/golden/*.json, each with the page
    passage it follows and its derivation written out),
  * invariants the definition implies (zero tables, zero factors, masks
    keeping exactly two of four, linearity in x, the clamp),
  * library routines on another route to the same number (scipy.sparse for
    the outliers, x (L R) computed as (x L) R, per-bucket sums for LUTs),
  * cross-format identities and brute force over every code and 2:4 pattern.
"""
from __future__ import annotations

import numpy as np
import scipy.sparse as sp

from golden_cases import golden_names, load_golden
from synth.layers import (
    LogicalLayer,
    PAIRS_2_4,
    bf16_bits_from_f32,
    draw_csr,
    draw_lut_codes,
    draw_mask_2_4,
    draw_mask_half,
    empty_csr,
)

REL = 1e-12


def _rng(seed):
    return np.random.default_rng(seed)


def _close(a, b, rel=REL):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    scale = max(1.0, float(np.abs(b).max(initial=0.0)))
    err = float(np.abs(a - b).max(initial=0.0))
    assert err <= rel * scale, f"max err {err:.3e} (scale {scale:.3e})"


def _lut_layer(seed, N=12, K=37, bits=3, csr=True):
    r = _rng(seed)
    codes, lut = draw_lut_codes(r, r, N, K, bits)
    rp, col, val = draw_csr(r, r, N, K, density=0.05) if csr else empty_csr(N)
    return LogicalLayer(K=K, N=N, dense=f"lut{bits}", codes=codes, lut=lut,
                        csr_row_ptr=rp, csr_col=col, csr_val=val)


def _x16(seed, M, K):
    return _rng(seed).normal(0, 1, size=(M, K)).astype(np.float16)


# ---------------------------------------------------------------------------
# worked examples
# ---------------------------------------------------------------------------

def pin_golden(O):
    for name in golden_names():
        layer, x, y_exp, _ = load_golden(name)
        y = O.forward(layer, x)
        assert np.array_equal(y, y_exp), f"{name}: {y} != {y_exp}"


def pin_bf16_decode(O):
    # 0x3F80 = 1, 0xC000 = -2, 0x3F81 = 1 + 2^-7, 0x0001 = 2^-133 (bf16 subnormal)
    layer = LogicalLayer(K=4, N=1, dense="lut3", codes=np.array([[1, 1, 1, 1]], np.uint8),
                         lut=np.array([[0, 1, 0, 0, 0, 0, 0, 0]], np.float16), x_dtype="bf16")
    x = np.array([[0x3F80, 0xC000, 0x3F81, 0x0001]], np.uint16)
    xp = O.activations(layer, x)
    assert np.array_equal(xp, np.array([[1.0, -2.0, 1.0 + 2.0 ** -7, 2.0 ** -133]]))


# ---------------------------------------------------------------------------
# invariants
# ---------------------------------------------------------------------------

def pin_zero_lut_is_csr_only(O):
    for bits in (3, 4):
        layer = _lut_layer(11 + bits, bits=bits)
        layer = layer.with_(lut=np.zeros_like(layer.lut))
        x = _x16(5, 3, layer.K)
        S = sp.csr_matrix((layer.csr_val.astype(np.float64), layer.csr_col, layer.csr_row_ptr),
                          shape=(layer.N, layer.K))
        y_lib = (S @ x.astype(np.float64).T).T
        _close(O.forward(layer, x), y_lib)


def pin_zero_factors_no_lowrank(O):
    layer = _lut_layer(21, N=9, K=33)
    x = _x16(6, 2, layer.K)
    base = O.forward(layer, x)
    r = 5
    for kind in ("fp16", "bf16", "int4"):
        if kind == "int4":
            lay = layer.with_(lr="int4", rank=r, group=16, L=np.zeros((layer.K, r), np.int8),
                              R=np.full((r, layer.N), 3, np.int8),
                              L_scale=np.full((3, r), 0.5, np.float16),
                              R_scale=np.full((1, layer.N), 0.25, np.float16))
        elif kind == "bf16":
            lay = layer.with_(lr="bf16", rank=r, L=np.zeros((layer.K, r), np.uint16),
                              R=bf16_bits_from_f32(np.ones((r, layer.N), np.float32)))
        else:
            lay = layer.with_(lr="fp16", rank=r, L=np.zeros((layer.K, r), np.float16),
                              R=np.ones((r, layer.N), np.float16))
        assert np.array_equal(O.forward(lay, x), base), kind
    # rank 0 is the same as no low-rank part
    assert np.array_equal(O.forward(layer.with_(lr="fp16", rank=0), x), base)


def pin_mask_2_4_keeps_two(O):
    r = _rng(31)
    N, K = 16, 64
    keep = draw_mask_2_4(r, N, K)
    q = r.choice(np.array([-8, -7, -3, -1, 1, 2, 5, 7], np.int8), size=(N, K))  # never 0
    layer = LogicalLayer(K=K, N=N, dense="int4", mask="2:4", qvals=q,
                         row_scale=np.full(N, 0.125, np.float16), keep=keep)
    D = O.dense_plane(layer)
    nz = (D != 0).reshape(N, K // 4, 4)
    assert (nz.sum(axis=2) == 2).all()
    assert np.array_equal(nz.reshape(N, K), keep.astype(bool))


def pin_linearity(O):
    layer = _lut_layer(41, N=10, K=50, bits=4)
    r = _rng(42)
    x1 = r.integers(-4, 5, size=(2, layer.K)).astype(np.float16)
    x2 = r.integers(-4, 5, size=(2, layer.K)).astype(np.float16)
    a, b = 0.5, -2.0
    xc = (a * x1.astype(np.float64) + b * x2.astype(np.float64)).astype(np.float16)
    _close(O.forward(layer, xc), a * O.forward(layer, x1) + b * O.forward(layer, x2))


def pin_clamp_identity_rows(O):
    # row n has weight 1 at column n only (lut[1] = 1, every other code 0):
    # y[m, n] must be the clamped activation x'[m, n].
    K = N = 6
    codes = np.zeros((N, K), np.uint8)
    codes[np.arange(N), np.arange(N)] = 1
    lut = np.zeros((N, 8), np.float16)
    lut[:, 1] = 1.0
    layer = LogicalLayer(K=K, N=N, dense="lut3", codes=codes, lut=lut, act_clamp=np.float16(1.5))
    x = np.array([[0.5, -3.0, 1.5, 2.0, -1.5, 100.0]], np.float16)
    assert np.array_equal(O.forward(layer, x), np.array([[0.5, -1.5, 1.5, 1.5, -1.5, 1.5]]))
    # no clamp: untouched
    assert np.array_equal(O.forward(layer.with_(act_clamp=None), x), x.astype(np.float64))


def pin_round_to_act_library(O):
    # Nearest-even rounding to the activation type against library casts:
    # numpy's float64 -> float16 and torch's float32 -> bfloat16.  Random values
    # over a wide exponent range (fp16 subnormals included) and exact midpoints
    # between neighbouring values of each type (the ties).
    import torch
    r = _rng(41)
    v = r.normal(0, 1, 4000) * np.exp2(r.integers(-26, 12, 4000))
    h = r.integers(1, 0x7BFE, 3000).astype(np.uint16)
    lo = h.view(np.float16).astype(np.float64)
    hi = (h + 1).view(np.float16).astype(np.float64)
    for vals in (v, (lo + hi) / 2, -(lo + hi) / 2):
        assert np.array_equal(O.round_to_act(vals, "f16"), vals.astype(np.float16).astype(np.float64))
    hb = r.integers(0x0081, 0x7F7E, 3000).astype(np.uint32) << 16
    lob = hb.view(np.float32).astype(np.float64)
    hib = (hb + (1 << 16)).view(np.float32).astype(np.float64)
    v32 = (r.normal(0, 1, 4000) * np.exp2(r.integers(-60, 60, 4000))).astype(np.float32).astype(np.float64)
    for vals in (v32, (lob + hib) / 2, -(lob + hib) / 2):
        ref = torch.tensor(vals, dtype=torch.float64).to(torch.float32).to(torch.bfloat16).to(torch.float64).numpy()
        assert np.array_equal(O.round_to_act(vals, "bf16"), ref)


def _int8_lr_layer(seed, K=24, N=5, rank=3):
    r = _rng(seed)
    q = r.integers(-31, 32, size=(N, K)).astype(np.int8)
    s = np.exp2(-r.integers(3, 7, size=N)).astype(np.float16)
    rp, col, val = draw_csr(r, r, N, K, density=0.2)
    L = (r.integers(-16, 17, size=(K, rank)) / 64).astype(np.float16)
    R = (r.integers(-16, 17, size=(rank, N)) / 64).astype(np.float16)
    return LogicalLayer(K=K, N=N, dense="int8", qvals=q, row_scale=s, csr_row_ptr=rp, csr_col=col,
                        csr_val=val, lr="fp16", rank=rank, L=L, R=R)


def pin_act_scale_identity(O):
    # factors of exactly 1 change nothing
    layer = _int8_lr_layer(51)
    x = _x16(52, 3, layer.K)
    ch = np.array([0, 5, 23], np.int32)
    scaled = layer.with_(xscale_ch=ch, xscale=np.ones(3, np.float16))
    assert np.array_equal(O.forward(scaled, x), O.forward(layer, x))


def pin_act_scale_equivalence(O):
    # SLiM's output-error variant keeps the product unchanged: weights of
    # input channel k times alpha_k, activations of channel k times 1/alpha_k.
    # With alpha a power of two every scaled value is exact, so the layer whose
    # column k of D and S and row k of L carry alpha_k, run with the factors
    # 1/alpha_k, must give the unscaled layer's output.
    ch = np.array([1, 7, 8, 20], np.int32)
    alpha = np.array([2.0, 4.0, 4.0, 2.0])
    for x_dtype in ("f16", "bf16"):
        layer = _int8_lr_layer(53).with_(x_dtype=x_dtype)
        r = _rng(54)
        xf = r.choice([-1.0, 1.0], size=(4, layer.K)) * r.uniform(0.5, 4.0, size=(4, layer.K))
        x = xf.astype(np.float16) if x_dtype == "f16" else bf16_bits_from_f32(xf.astype(np.float32))
        q = layer.qvals.astype(np.int64)
        q[:, ch] *= alpha.astype(np.int64)[None, :]          # |q| <= 31, so 4q still fits int8
        val = layer.csr_val.astype(np.float64)
        L = layer.L.astype(np.float64)
        for j, k in enumerate(ch):
            val[layer.csr_col == k] *= alpha[j]
            L[k] *= alpha[j]
        scaled = layer.with_(qvals=q.astype(np.int8), csr_val=val.astype(np.float16), L=L.astype(np.float16),
                             xscale_ch=ch, xscale=(1.0 / alpha).astype(np.float16))
        assert np.isin(layer.csr_col, ch).any()
        _close(O.forward(scaled, x), O.forward(layer, x))


# ---------------------------------------------------------------------------
# library routines on another route
# ---------------------------------------------------------------------------

def _lowrank_lib(layer):
    """L_hat, R_hat built with np.repeat over the group scales (not the oracle's indexing)."""
    if layer.lr == "int4":
        g = layer.group
        Ls = np.repeat(layer.L_scale.astype(np.float64), g, axis=0)[: layer.K]
        Rs = np.repeat(layer.R_scale.astype(np.float64), g, axis=0)[: layer.rank]
        return layer.L.astype(np.float64) * Ls, layer.R.astype(np.float64) * Rs
    if layer.lr == "bf16":
        to = lambda b: (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        return to(layer.L), to(layer.R)
    return layer.L.astype(np.float64), layer.R.astype(np.float64)


def _library_forward(layer, x64):
    """x D^T (bucket sums for LUTs) + S x (scipy) + (x L) R."""
    N, K = layer.N, layer.K
    if layer.dense.startswith("lut"):
        nb = 1 << layer.bits
        lut = layer.lut.astype(np.float64)
        # y[m, n] = sum_c lut[n, c] * (sum of x[m, k] over k with code[n, k] == c)
        onehot = (layer.codes[:, :, None] == np.arange(nb)[None, None, :]).astype(np.float64)  # [N,K,nb]
        buckets = np.einsum("mk,nkc->mnc", x64, onehot)
        yd = np.einsum("mnc,nc->mn", buckets, lut)
    else:
        q = layer.qvals.astype(np.float64)
        if layer.mask != "none":
            q = q * layer.keep.astype(np.float64)
        yd = (x64 @ q.T) * layer.row_scale.astype(np.float64)[None, :]
    y = yd
    if layer.csr_col is not None and layer.nnz:
        S = sp.csr_matrix((layer.csr_val.astype(np.float64), layer.csr_col, layer.csr_row_ptr), shape=(N, K))
        y = y + (S @ x64.T).T
    if layer.lr != "none" and layer.rank:
        Lh, Rh = _lowrank_lib(layer)
        y = y + (x64 @ Lh) @ Rh
    return y


def pin_library_route(O):
    for bits in (3, 4):
        layer = _lut_layer(50 + bits, N=13, K=45, bits=bits)
        x = _x16(51, 3, layer.K)
        _close(O.forward(layer, x), _library_forward(layer, x.astype(np.float64)), rel=1e-12)
    # integer + masks + low-rank (int4 groups with a ragged last group, non-square)
    r = _rng(60)
    N, K, rank, g = 11, 40, 3, 16
    keep = draw_mask_2_4(r, N, K)
    q = r.integers(-8, 8, size=(N, K)).astype(np.int8)
    rp, col, val = draw_csr(r, r, N, K, density=0.1)
    layer = LogicalLayer(K=K, N=N, dense="int4", mask="2:4", qvals=q, keep=keep,
                         row_scale=r.uniform(0.01, 0.1, N).astype(np.float16),
                         csr_row_ptr=rp, csr_col=col, csr_val=val, lr="int4", rank=rank, group=g,
                         L=r.integers(-8, 8, size=(K, rank)).astype(np.int8),
                         R=r.integers(-8, 8, size=(rank, N)).astype(np.int8),
                         L_scale=r.uniform(0.01, 0.1, size=(3, rank)).astype(np.float16),
                         R_scale=r.uniform(0.01, 0.1, size=(1, N)).astype(np.float16))
    x = _x16(61, 4, K)
    _close(O.forward(layer, x), _library_forward(layer, x.astype(np.float64)))
    # int8 + bitmap + bf16 factors + bf16 activations
    keep = draw_mask_half(r, N, K)
    q8 = r.integers(-127, 128, size=(N, K)).astype(np.int8)
    layer8 = LogicalLayer(K=K, N=N, dense="int8", mask="bitmap", qvals=q8, keep=keep,
                          row_scale=r.uniform(0.001, 0.01, N).astype(np.float16),
                          lr="bf16", rank=rank,
                          L=bf16_bits_from_f32(r.normal(0, 0.1, (K, rank))),
                          R=bf16_bits_from_f32(r.normal(0, 0.1, (rank, N))), x_dtype="bf16")
    xb = bf16_bits_from_f32(r.normal(0, 1, (2, K)))
    xb64 = (xb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    _close(O.forward(layer8, xb), _library_forward(layer8, xb64))


def pin_lowrank_groups_ragged(O):
    # K = 130 with group 128: rows 0..127 take scale row 0, rows 128, 129 take scale row 1
    K, r = 130, 2
    Lq = np.ones((K, r), np.int8)
    Ls = np.array([[0.5, 2.0], [4.0, 0.25]], np.float16)
    Rq = np.array([[1], [-2]], np.int8)       # r = 2 rows; one group of 128 along r
    Rs = np.array([[0.125]], np.float16)
    layer = LogicalLayer(K=K, N=1, dense="lut3", codes=np.zeros((1, K), np.uint8),
                         lut=np.zeros((1, 8), np.float16), lr="int4", rank=r, group=128,
                         L=Lq, R=Rq, L_scale=Ls, R_scale=Rs)
    Lh, Rh = O.lowrank_factors(layer)
    assert np.array_equal(Lh[:128], np.tile([0.5, 2.0], (128, 1)))
    assert np.array_equal(Lh[128:], np.tile([4.0, 0.25], (2, 1)))
    assert np.array_equal(Rh, np.array([[0.125], [-0.25]]))
    # x = e_129 selects row 129 of L_hat: y = 4*0.125 + 0.25*(-0.25) = 0.4375
    x = np.zeros((1, K), np.float16)
    x[0, 129] = 1
    assert np.array_equal(O.forward(layer, x), np.array([[0.4375]]))


# ---------------------------------------------------------------------------
# cross-format identities and brute force
# ---------------------------------------------------------------------------

def pin_lut4_equals_int4(O):
    r = _rng(70)
    N, K = 9, 24
    codes = r.integers(0, 16, size=(N, K)).astype(np.uint8)
    # scales with at most 7 significant bits, so that (c - 8) * s is exact in fp16
    s = (r.integers(1, 128, N) * 2.0 ** -12).astype(np.float16)
    lut = ((np.arange(16)[None, :] - 8) * s.astype(np.float64)[:, None]).astype(np.float16)
    lut_layer = LogicalLayer(K=K, N=N, dense="lut4", codes=codes, lut=lut)
    int_layer = LogicalLayer(K=K, N=N, dense="int4", qvals=(codes.astype(np.int16) - 8).astype(np.int8),
                             row_scale=s)
    x = _x16(71, 2, K)
    _close(O.forward(lut_layer, x), O.forward(int_layer, x))


def pin_2_4_equals_bitmap(O):
    r = _rng(80)
    N, K = 7, 32
    keep = draw_mask_2_4(r, N, K)
    q = r.integers(-8, 8, size=(N, K)).astype(np.int8)
    s = r.uniform(0.01, 0.1, N).astype(np.float16)
    a = LogicalLayer(K=K, N=N, dense="int4", mask="2:4", qvals=q, keep=keep, row_scale=s)
    b = LogicalLayer(K=K, N=N, dense="int8", mask="bitmap", qvals=q, keep=keep, row_scale=s)
    x = _x16(81, 3, K)
    assert np.array_equal(O.forward(a, x), O.forward(b, x))


def pin_brute_force_codes_and_patterns(O):
    # every code at every position of a 1x10 (3-bit) and 1x16 (4-bit) row
    for bits, K in ((3, 10), (4, 16)):
        nb = 1 << bits
        lut = (np.arange(nb, dtype=np.float64) * 0.25 - 1.0).astype(np.float16)[None, :]
        for c in range(nb):
            for k in range(K):
                codes = np.zeros((1, K), np.uint8)
                codes[0, k] = c
                D = O.dense_plane(LogicalLayer(K=K, N=1, dense=f"lut{bits}", codes=codes, lut=lut))
                expect = np.full(K, float(lut[0, 0]))
                expect[k] = float(lut[0, c])
                assert np.array_equal(D[0], expect), (bits, c, k)
    # all 6 x 6 two-of-four patterns on a K = 8 row
    q = np.array([[1, 2, 3, 4, 5, 6, 7, -8]], np.int8)
    for p0 in range(6):
        for p1 in range(6):
            keep = np.zeros((1, 8), np.uint8)
            keep[0, PAIRS_2_4[p0]] = 1
            keep[0, 4 + PAIRS_2_4[p1]] = 1
            layer = LogicalLayer(K=8, N=1, dense="int4", mask="2:4", qvals=q, keep=keep,
                                 row_scale=np.array([1.0], np.float16))
            D = O.dense_plane(layer)
            assert np.array_equal(D[0], np.where(keep[0] == 1, q[0], 0).astype(np.float64))


def pin_debug_planes(O):
    # LUT planes hold the centroids exactly; S16 holds the outliers at their positions;
    # integer planes are q*s rounded once to fp16 (7 * fp16(0.02/7) = 0.0200004... -> fp16)
    layer, x, _, _ = load_golden("lut3_csr_2x10")
    D16, S16, L32, R32 = O.debug_planes(layer)
    assert D16.dtype == np.float16 and L32 is None
    assert np.array_equal(D16[0], np.array([-1, -0.5, -0.25, 0, 0.25, 0.5, 1, 2, -1, 2], np.float16))
    S_expect = np.zeros((2, 10), np.float16)
    S_expect[0, 1], S_expect[1, 0], S_expect[1, 9] = 0.5, -0.25, 1.5
    assert np.array_equal(S16, S_expect)
    s = np.float16(0.02 / 7)                           # 0x19DA
    assert s.view(np.uint16) == 0x19DA
    layer = LogicalLayer(K=2, N=1, dense="int4", qvals=np.array([[7, -8]], np.int8),
                         row_scale=np.array([s], np.float16))
    D16, _, _, _ = O.debug_planes(layer)
    # 7 * 0.002857208251953125 = 0.020000457763671875; nearest fp16 is 0x251F = 0.0200042724609375
    # -8 * s = -0.022857666015625 is exact in fp16 (0xA5DA)
    assert D16.view(np.uint16).tolist() == [[0x251F, 0xA5DA]]
    g, _, _, _ = load_golden("int4_2of4_lr_int4_2x8")
    _, _, L32, R32 = O.debug_planes(g)
    assert L32.dtype == np.float32 and np.array_equal(L32[:, 0], np.array([0.5, 0, 0, 0, 0, 0, 0, -1], np.float32))
    assert np.array_equal(R32, np.array([[0.5, -0.5]], np.float32))


def pin_row_subset(O):
    layer = _lut_layer(90, N=20, K=31)
    x = _x16(91, 2, layer.K)
    rows = [19, 0, 7, 7, 3]
    full = O.forward(layer, x)
    assert np.array_equal(O.forward(layer, x, rows=rows), full[:, rows])


def pin_bound(O):
    layer, x, _, _ = load_golden("lut3_csr_2x10")
    B = O.bound(layer, x)
    # |W| row 0 = |dense| with col 1 dense -0.5 plus outlier 0.5 -> 0; |x0| = [1,2,1,0,1,2,1,1,1,2]
    # row 0 |W| = [1,0,0.25,0,0.25,0.5,1,2,1,2]: sum |x||W| = 1+0+0.25+0+0.25+1+1+2+1+4 = 10.5
    assert abs(B[0, 0] - 10.5e-3) < 1e-15
    # row 1 |W| = [0.875-0.25, 0.75, 0.625, 0.5, 0.375, 0.25, 0.125, 0, 0.125, 0.125+1.5]
    # dot |x0| = 0.625+1.5+0.625+0+0.375+0.5+0.125+0+0.125+3.25 = 7.125
    assert abs(B[0, 1] - 7.125e-3) < 1e-15


def pin_forward_and_bound(O):
    """forward_and_bound, the checker of every GPU parity test, against hand values and the pinned pair."""
    # lut4_lr_bf16_2x4: W_hat = D + (L R)^T with (L R)^T rows [2, 0.5, 1, 0.125] and [-1, 3, -0.5, 0.75]:
    # W_hat row 0 = [-2+2, 1.75+0.5, 0+1, -1+0.125] = [0, 2.25, 1, -0.875],
    # row 1 = [-1/16-1, 2/16+3, -3/16-0.5, -15/16+0.75] = [-1.0625, 3.125, -0.6875, -0.1875];
    # |x| = [1, 2, 0.5, 4]: bound row 0 = 1e-3 (0 + 4.5 + 0.5 + 3.5) = 8.5e-3,
    # row 1 = 1e-3 (1.0625 + 6.25 + 0.34375 + 0.75) = 8.40625e-3
    layer, x, y_exp, _ = load_golden("lut4_lr_bf16_2x4")
    y, B = O.forward_and_bound(layer, x)
    assert np.array_equal(y, y_exp), f"{y} != {y_exp}"
    assert abs(B[0, 0] - 8.5e-3) < 1e-15 and abs(B[0, 1] - 8.40625e-3) < 1e-15, B
    # lut3_csr_2x10: the hand bound of pin_bound
    layer, x, y_exp, _ = load_golden("lut3_csr_2x10")
    y, B = O.forward_and_bound(layer, x)
    assert np.array_equal(y, y_exp)
    assert abs(B[0, 0] - 10.5e-3) < 1e-15 and abs(B[0, 1] - 7.125e-3) < 1e-15, B
    # every worked example: the hand-derived outputs
    for name in golden_names():
        layer, x, y_exp, _ = load_golden(name)
        y, B = O.forward_and_bound(layer, x)
        assert np.array_equal(y, y_exp), name
        assert (B >= 0).all(), name
    # random layers of every format, both activation types, with clamps and rank terms: the same
    # numbers as the separately pinned forward and bound, bit for bit, on a row subset too
    r = _rng(123)
    for seed, (dense, mask, lr, xd) in enumerate([("lut3", "none", "fp16", "f16"), ("lut4", "none", "bf16", "bf16"),
                                                  ("int4", "2:4", "int4", "f16"), ("int8", "bitmap", "none", "bf16"),
                                                  ("int4", "none", "none", "f16"), ("int8", "none", "fp16", "f16")]):
        N, K, rk = 7, 24, 3
        kw = dict(K=K, N=N, dense=dense, mask=mask, x_dtype=xd)
        if dense.startswith("lut"):
            codes, lut = draw_lut_codes(r, r, N, K, int(dense[3]))
            kw.update(codes=codes, lut=lut)
        else:
            lo = -8 if dense == "int4" else -127
            kw.update(qvals=r.integers(lo, -lo, size=(N, K)).astype(np.int8),
                      row_scale=(r.random(N) * 0.05 + 0.01).astype(np.float16))
            if mask == "2:4":
                kw["keep"] = draw_mask_2_4(r, N, K)
            elif mask == "bitmap":
                kw["keep"] = draw_mask_half(r, N, K)
        rp, col, val = draw_csr(r, r, N, K, density=0.1)
        kw.update(csr_row_ptr=rp, csr_col=col, csr_val=val)
        if lr == "int4":
            kw.update(lr="int4", rank=rk, group=8, L=r.integers(-8, 8, size=(K, rk)).astype(np.int8),
                      R=r.integers(-8, 8, size=(rk, N)).astype(np.int8),
                      L_scale=(r.random((3, rk)) * 0.1).astype(np.float16),
                      R_scale=(r.random((1, N)) * 0.1).astype(np.float16))
        elif lr == "bf16":
            kw.update(lr="bf16", rank=rk, L=bf16_bits_from_f32(r.normal(0, 0.1, (K, rk)).astype(np.float32)),
                      R=bf16_bits_from_f32(r.normal(0, 0.1, (rk, N)).astype(np.float32)))
        elif lr == "fp16":
            kw.update(lr="fp16", rank=rk, L=r.normal(0, 0.1, (K, rk)).astype(np.float16),
                      R=r.normal(0, 0.1, (rk, N)).astype(np.float16))
        if seed % 2:
            kw["act_clamp"] = np.float16(1.5)
        layer = LogicalLayer(**kw)
        xf = r.normal(0, 1, (3, K)).astype(np.float32)
        x = bf16_bits_from_f32(xf) if xd == "bf16" else xf.astype(np.float16)
        for rows in (None, [6, 0, 3]):
            y, B = O.forward_and_bound(layer, x, rows)
            assert np.array_equal(y, O.forward(layer, x, rows)), (dense, mask, lr, xd, rows)
            assert np.array_equal(B, O.bound(layer, x, rows)), (dense, mask, lr, xd, rows)


ALL_PINS = [
    pin_golden,
    pin_bf16_decode,
    pin_zero_lut_is_csr_only,
    pin_zero_factors_no_lowrank,
    pin_mask_2_4_keeps_two,
    pin_linearity,
    pin_clamp_identity_rows,
    pin_round_to_act_library,
    pin_act_scale_identity,
    pin_act_scale_equivalence,
    pin_library_route,
    pin_lowrank_groups_ragged,
    pin_lut4_equals_int4,
    pin_2_4_equals_bitmap,
    pin_brute_force_codes_and_patterns,
    pin_debug_planes,
    pin_row_subset,
    pin_bound,
    pin_forward_and_bound,
]


def failing_pins(O):
    bad = []
    for p in ALL_PINS:
        try:
            p(O)
        except Exception as e:  # noqa: BLE001 -- a mutant may raise anything
            bad.append((p.__name__, repr(e)[:200]))
    return bad
