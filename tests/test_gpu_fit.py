"""The data-free LUT packer (cl_fit_lut) against its CPU oracle, through the C
ABI (needs an MI355X).

Bit for bit: codes, LUTs, CSR row pointers, columns and values, at sizes the
oracle runs in seconds (ragged K, ties at the outlier threshold, rows that are
all outliers, no outliers, one iteration).  At a LLaMA layer's full size: the
outlier set's defining properties over the whole matrix and the k-means,
LUT and codes of sampled rows against the oracle.  End to end: the fitted
layer packed and run through the forward matches the oracle's forward of it.
"""
import sys

import numpy as np
import pytest

import compressed_linear_amd as cla
from oracle import fit_oracle as F
from gpu_util import check_bound, gpu_forward, torch_cuda
from synth.layers import LogicalLayer, bf16_bits_from_f32, make_layer, make_x

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def _weights(seed, N, K, tail=0.003):
    r = np.random.default_rng(seed)
    w = r.normal(0, 0.02, (N, K))
    big = r.random((N, K)) < tail
    w = np.where(big, r.normal(0, 0.3, (N, K)), w)
    return w.astype(np.float16)


def _gpu_fit(W, bits, n_out, iters):
    torch = torch_cuda()
    Wd = torch.from_numpy(W.view(np.int16)).view(torch.float16).cuda()
    codes, lut, rp, col, val = cla.fit_lut(Wd, bits, n_out, iters)
    torch.cuda.synchronize()
    return (codes.cpu().numpy(), lut.cpu().numpy(), rp.cpu().numpy(), col.cpu().numpy(), val.cpu().numpy())


def _same(g, o, what):
    names = ["codes", "lut", "row_ptr", "col", "val"]
    for nm, a, b in zip(names, g, o):
        a = np.asarray(a)
        b = np.asarray(b)
        if a.dtype == np.float16:
            a, b = a.view(np.uint16), b.view(np.uint16)
        assert a.shape == b.shape and np.array_equal(a, b), f"{what}: {nm} differs at {np.argwhere(a != b)[:5]}"


@pytest.mark.parametrize("N,K,bits,frac,iters", [(130, 1000, 3, 0.0045, 50), (70, 777, 4, 0.01, 50),
                                                 (33, 37, 3, 0.05, 50), (5, 1, 4, 0.0, 50), (40, 300, 4, 0.0045, 1),
                                                 (300, 4096, 4, 0.0045, 30)])
def test_fit_bit_exact(N, K, bits, frac, iters):
    W = _weights(N * 7 + K, N, K)
    n_out = int(round(frac * N * K))
    say("fit", N, K, bits, n_out, iters)
    _same(_gpu_fit(W, bits, n_out, iters), F.fit_lut(W, bits, n_out, iters), f"{N}x{K} b{bits}")


def test_fit_ties_and_degenerate_rows():
    r = np.random.default_rng(3)
    # few distinct magnitudes: many ties at the threshold, split across rows
    W = r.choice(np.array([-0.5, -0.25, 0.0, 0.125, 0.25, 0.5], np.float16), size=(60, 260))
    W[7] = np.float16(0.0)            # a row of zeros (and -0)
    W[8, ::2] = np.float16(-0.0)
    W[9] = np.float16(0.5)            # a row that becomes all outliers
    for n_out in (0, 1, 260 + 17, 3000, 60 * 260):
        say("ties", n_out)
        _same(_gpu_fit(W, 3, n_out, 40), F.fit_lut(W, 3, n_out, 40), f"ties n_out={n_out}")


def test_fit_rejects_bad_input():
    torch = torch_cuda()
    W = _weights(5, 8, 64)
    W[3, 3] = np.float16(9000.0)
    with pytest.raises(cla.ClError):
        _gpu_fit(W, 3, 4, 10)
    Wd = torch.zeros((4, 40000), dtype=torch.float16, device="cuda")
    with pytest.raises(cla.ClError):
        cla.fit_lut(Wd, 3, 1, 10)
    with pytest.raises(cla.ClError):
        cla.fit_lut(torch.zeros((4, 64), dtype=torch.float16, device="cuda"), 5, 1, 10)


def test_fit_full_size_properties_and_sampled_rows():
    # LLaMA-7B gate projection shape, 0.45 % outliers, 4-bit
    N, K, bits = 11008, 4096, 4
    W = _weights(11, N, K)
    n_out = int(round(0.0045 * N * K))
    say("fit full size", N, K, n_out)
    codes, lut, rp, col, val = _gpu_fit(W, bits, n_out, 30)
    assert rp[0] == 0 and rp[-1] == n_out and np.all(np.diff(rp) >= 0)
    out = np.zeros((N, K), bool)
    rows = np.repeat(np.arange(N), np.diff(rp))
    out[rows, col] = True
    assert out.sum() == n_out
    for n in np.random.default_rng(1).choice(N, 40, replace=False):
        assert np.all(np.diff(col[rp[n]:rp[n + 1]]) > 0)
    a = np.abs(W.astype(np.float64))
    thr = a[out].min()
    assert thr >= a[~out].max()
    # ties at the threshold: the outliers among them have the lowest indices
    tie = np.flatnonzero((a == thr).ravel())
    chosen = out.ravel()[tie]
    assert np.all(chosen[:chosen.sum()]) and not np.any(chosen[chosen.sum():])
    # sampled rows: k-means, LUT, codes and outlier values against the oracle
    for n in np.random.default_rng(2).choice(N, 24, replace=False):
        dense = ~out[n]
        c = F.kmeans_row(W[n, dense], 1 << bits, 30)
        l16 = F.round_to_f16(c).astype(np.float16)
        assert np.array_equal(lut[n].view(np.uint16), l16.view(np.uint16)), n
        w = W[n].astype(np.float64)
        assert np.array_equal(codes[n], F.nearest_code(np.where(dense, w, 0.0), l16)), n
        c0 = F.nearest_code(np.array([0.0]), l16)[0]
        want = F.round_to_f16(w[col[rp[n]:rp[n + 1]]] - float(l16[c0])).astype(np.float16)
        assert np.array_equal(val[rp[n]:rp[n + 1]].view(np.uint16), want.view(np.uint16)), n


def test_fit_then_forward():
    # the fitted arrays are a LUT layer with CSR outliers: pack, create, forward
    N, K = 300, 1024
    W = _weights(21, N, K)
    codes, lut, rp, col, val = _gpu_fit(W, 4, int(0.0045 * N * K), 40)
    layer = LogicalLayer(K=K, N=N, dense="lut4", codes=codes, lut=lut, csr_row_ptr=rp, csr_col=col, csr_val=val)
    x = np.random.default_rng(4).normal(0, 1, (3, K)).astype(np.float16)
    y = gpu_forward(layer, x)
    check_bound(y, layer, x, what="fitted layer")
    # and the fitted layer approximates the original weights
    y_w = x.astype(np.float64) @ W.astype(np.float64).T
    assert np.linalg.norm(y - y_w) < 0.2 * np.linalg.norm(y_w)


# ---------------------------------------------------------------------------
# integer formats (cl_fit_int)
# ---------------------------------------------------------------------------

OMASK = {"none": "none", "2:4": "2:4", "bitmap": "half"}


def _gpu_fit_int(W, bits, mask, grid):
    torch = torch_cuda()
    Wd = torch.from_numpy(W.view(np.int16)).view(torch.float16).cuda()
    q, s, keep = cla.fit_int(Wd, bits, mask, grid)
    torch.cuda.synchronize()
    return q.cpu().numpy(), s.cpu().numpy(), None if keep is None else keep.cpu().numpy()


@pytest.mark.parametrize("N,K,bits,mask,grid", [(40, 256, 4, "2:4", 20), (30, 333, 8, "bitmap", 12),
                                                (25, 100, 4, "none", 50), (9, 1, 8, "bitmap", 5),
                                                (12, 1000, 8, "none", 3), (16, 64, 4, "2:4", 1)])
def test_fit_int_bit_exact(N, K, bits, mask, grid):
    W = _weights(N * 3 + K, N, K, tail=0.02)
    say("fit int", N, K, bits, mask, grid)
    q, s, keep = _gpu_fit_int(W, bits, mask, grid)
    oq, os_, ok = F.fit_int(W, bits, OMASK[mask], grid)
    assert np.array_equal(s.view(np.uint16), os_.view(np.uint16)), np.argwhere(s.view(np.uint16) != os_.view(np.uint16))[:5]
    assert np.array_equal(q, oq)
    if keep is not None:
        assert np.array_equal(keep, ok)


def test_fit_int_ties_and_degenerate_rows():
    r = np.random.default_rng(8)
    W = r.choice(np.array([-0.5, -0.25, 0.0, 0.125, 0.25, 0.5], np.float16), size=(20, 96))
    W[3] = np.float16(0.0)
    W[4, ::3] = np.float16(-0.0)
    for bits, mask in ((4, "2:4"), (8, "bitmap"), (4, "none")):
        say("fit int ties", bits, mask)
        q, s, keep = _gpu_fit_int(W, bits, mask, 16)
        oq, os_, ok = F.fit_int(W, bits, OMASK[mask], 16)
        assert np.array_equal(s.view(np.uint16), os_.view(np.uint16)) and np.array_equal(q, oq)
        if keep is not None:
            assert np.array_equal(keep, ok)


def test_fit_int_full_size_properties_and_sampled_rows():
    # SLiM-style INT4 2:4 at the up projection's shape (4096 -> 11008)
    N, K = 11008, 4096
    W = _weights(13, N, K, tail=0.002)
    say("fit int full size")
    q, s, keep = _gpu_fit_int(W, 4, "2:4", 100)
    assert np.all(keep.reshape(N, K // 4, 4).sum(axis=2) == 2)
    assert np.abs(q).max() <= 7 and not q[keep == 0].any()
    for n in np.random.default_rng(3).choice(N, 3, replace=False):
        ok = F.magnitude_mask(W[n:n + 1], "2:4")[0]
        assert np.array_equal(keep[n], ok)
        os_, oq = F.clip_search_row(W[n], ok.astype(bool), 4, 100)
        assert s[n].view(np.uint16) == np.float16(os_).view(np.uint16) and np.array_equal(q[n], oq), n


def test_fit_int_then_forward():
    N, K = 260, 1024
    W = _weights(31, N, K)
    q, s, keep = _gpu_fit_int(W, 4, "2:4", 60)
    layer = LogicalLayer(K=K, N=N, dense="int4", mask="2:4", qvals=q, row_scale=s, keep=keep)
    x = np.random.default_rng(5).normal(0, 1, (4, K)).astype(np.float16)
    y = gpu_forward(layer, x)
    check_bound(y, layer, x, what="fitted int4 2:4 layer")
    q8, s8, k8 = _gpu_fit_int(W, 8, "bitmap", 60)
    layer8 = LogicalLayer(K=K, N=N, dense="int8", mask="bitmap", qvals=q8, row_scale=s8, keep=k8)
    y8 = gpu_forward(layer8, x)
    check_bound(y8, layer8, x, what="fitted int8 bitmap layer")


# ---------------------------------------------------------------------------
# AbsMax int4 groups of the low-rank factors (cl_quant_absmax)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("R,C,g", [(4096, 128, 128), (1000, 70, 128), (37, 5, 8), (9, 300, 1), (11008, 64, 128)])
def test_quant_absmax_bit_exact(dtype, R, C, g):
    torch = torch_cuda()
    r = np.random.default_rng(R + C + g)
    x = r.normal(0, 0.01, (R, C))
    x[: min(g, R), 0] = 0.0  # an all-zero group
    if dtype == "bf16":
        bits = bf16_bits_from_f32(x.astype(np.float32))
        Fd = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()
        host = bits
    else:
        host = x.astype(np.float16)
        Fd = torch.from_numpy(host).cuda()
    say("absmax", dtype, R, C, g)
    q, sc = cla.quant_absmax(Fd, g)
    torch.cuda.synchronize()
    oq, osc = F.absmax_groups(host, g, dtype)
    assert np.array_equal(sc.cpu().numpy().view(np.uint16), osc.view(np.uint16))
    assert np.array_equal(q.cpu().numpy(), oq)


def test_quant_absmax_then_forward():
    # rank-64 factors quantized on the GPU feed an int4 low-rank layer
    torch = torch_cuda()
    r = np.random.default_rng(9)
    base = make_layer(3, 1, K=768, N=130)
    Lf = r.normal(0, 0.01, (768, 64)).astype(np.float16)
    Rf = r.normal(0, 0.01, (64, 130)).astype(np.float16)
    Lq, Ls = cla.quant_absmax(torch.from_numpy(Lf).cuda(), 128)
    Rq, Rs = cla.quant_absmax(torch.from_numpy(Rf).cuda(), 128)
    layer = base.with_(lr="int4", rank=64, group=128, L=Lq.cpu().numpy(), R=Rq.cpu().numpy(),
                       L_scale=Ls.cpu().numpy(), R_scale=Rs.cpu().numpy())
    x = make_x(3, 1, 8, K=768)
    check_bound(gpu_forward(layer, x), layer, x, what="int4 factors quantized on the GPU")


def test_fit_longest_rows():
    # K = 28672 (LLaMA-70B down projection's rows): the largest row the packers take
    N, K = 24, 28672
    W = _weights(17, N, K)
    say("fit long rows")
    _same(_gpu_fit(W, 3, int(0.0045 * N * K), 12), F.fit_lut(W, 3, int(0.0045 * N * K), 12), "K=28672 lut3")
    q, s, keep = _gpu_fit_int(W[:6], 8, "bitmap", 4)
    oq, os_, ok = F.fit_int(W[:6], 8, "half", 4)
    assert np.array_equal(s.view(np.uint16), os_.view(np.uint16)) and np.array_equal(q, oq) and np.array_equal(keep, ok)
