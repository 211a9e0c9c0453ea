"""Host packer: lossless layout, validation, byte accounting (no GPU)."""
import numpy as np
import pytest

import compressed_linear_amd as cla
from blob_unpack import unpack
from golden_cases import golden_names, load_golden
from synth.layers import LogicalLayer, draw_csr, draw_csr_skewed, draw_mask_2_4, draw_mask_half, make_layer


def _roundtrip(layer):
    blob, acct = cla.pack(layer)
    h, u = unpack(blob)
    assert (h["K"], h["N"]) == (layer.K, layer.N)
    if layer.dense.startswith("lut"):
        assert np.array_equal(u["codes"], layer.codes)
        assert np.array_equal(u["lut"].view(np.uint16), layer.lut.view(np.uint16))
    else:
        keep = np.ones((layer.N, layer.K), bool) if layer.mask == "none" else layer.keep.astype(bool)
        if layer.mask != "none":
            assert np.array_equal(u["keep"].astype(bool), keep)
        assert np.array_equal(np.where(keep, u["qvals"], 0), np.where(keep, layer.qvals, 0))
        assert np.array_equal(u["row_scale"].view(np.uint16), layer.row_scale.view(np.uint16))
    if layer.nnz:
        assert np.array_equal(u["csr_row_ptr"], layer.csr_row_ptr)
        assert np.array_equal(u["csr_col"], layer.csr_col)
        assert np.array_equal(u["csr_val"].view(np.uint16), layer.csr_val.view(np.uint16))
    if layer.lr != "none" and layer.rank:
        if layer.lr == "int4":
            assert np.array_equal(u["L"], layer.L) and np.array_equal(u["R"], layer.R)
            assert np.array_equal(u["L_scale"].view(np.uint16), layer.L_scale.view(np.uint16))
            assert np.array_equal(u["R_scale"].view(np.uint16), layer.R_scale.view(np.uint16))
        else:
            b = lambda a: np.asarray(a).view(np.uint16)
            assert np.array_equal(u["L"], b(layer.L)) and np.array_equal(u["R"], b(layer.R))
    ch = layer.xscale_ch
    assert h["n_xscale"] == (0 if ch is None else len(ch))
    if ch is not None and len(ch):
        dense = np.ones(layer.K, np.float16)
        dense[ch] = layer.xscale
        assert np.array_equal(u["xscale_dense"].view(np.uint16), dense.view(np.uint16))
        assert acct["act_scale"] == 6 * len(ch)
    else:
        assert acct["act_scale"] == 0 and "xscale" not in h["sections"]
    assert acct["total"] == sum(acct[f] for f in ("codes", "lut_or_scale", "mask_meta", "csr", "lowrank", "act_scale"))
    return blob, acct


@pytest.mark.parametrize("name", golden_names())
def test_roundtrip_golden(name):
    layer, _, _, _ = load_golden(name)
    _roundtrip(layer)


@pytest.mark.parametrize("cfg,K,N", [(1, 1000, 130), (2, 999 + 1, 70), (3, 512, 100), (4, 640, 66), (5, 1210, 129)])
def test_roundtrip_configs(cfg, K, N):
    _roundtrip(make_layer(cfg, 0, K=K, N=N))


@pytest.mark.parametrize("cfg,K,N", [(2, 1000, 70), (4, 640, 66), (5, 1210, 129)])
def test_roundtrip_act_scale(cfg, K, N):
    from synth.layers import with_act_scale
    lay = with_act_scale(make_layer(cfg, 0, K=K, N=N), frac=0.05)
    _, acct = _roundtrip(lay)
    _, acct0 = cla.pack(lay.with_(xscale_ch=None, xscale=None))
    assert acct["total"] == acct0["total"] + 6 * len(lay.xscale_ch)


def test_roundtrip_int4_plain_and_int8_plain():
    r = np.random.default_rng(3)
    for dense, lo, hi in (("int4", -8, 8), ("int8", -127, 128)):
        for K in (1, 31, 33, 100):
            q = r.integers(lo, hi, size=(5, K)).astype(np.int8)
            lay = LogicalLayer(K=K, N=5, dense=dense, qvals=q, row_scale=np.full(5, 0.5, np.float16))
            _roundtrip(lay)


def test_roundtrip_lut3_every_position():
    # every code at every position of a row; ragged K around the 10-per-word boundary
    for K in (1, 9, 10, 11, 39, 40, 41, 81):
        codes = (np.arange(8 * K).reshape(8, K) % 8).astype(np.uint8)
        codes = np.roll(codes, 3, axis=1)
        lay = LogicalLayer(K=K, N=8, dense="lut3", codes=codes, lut=np.zeros((8, 8), np.float16))
        _roundtrip(lay)


def test_accounting_closed_forms():
    # LUT3 4096x4096 + 0.45% CSR (the 4096 x 4096 layer of the 3-bit workload)
    lay = make_layer(1, 0)
    _, acct = cla.pack(lay)
    assert acct["codes"] == 4096 * 410 * 4
    assert acct["lut_or_scale"] == 4096 * 8 * 2
    assert acct["csr"] == 6 * lay.nnz + 4 * 4097
    assert acct["total"] == 7252346
    # INT4 2:4 + int4 r128 (11008 x 4096)
    lay3 = make_layer(3, 0, K=4096, N=11008)
    _, a3 = cla.pack(lay3)
    assert a3["codes"] + a3["mask_meta"] + a3["lut_or_scale"] == 16930304
    assert a3["lowrank"] == 996864


def test_bits_per_weight_matches_page_figure():
    """SqueezeLLM page, Key results: 3-bit codes with 0.45% sparse outliers average 3.24 bits.

    With ideal 3-bit packing (codes 3 bits, 8 fp16 centroids per 4096-wide row,
    48 bits per outlier: 16-bit value + 32-bit column, plus row pointers) the
    packer's accounting gives 3.255 bits; the 10-per-word layout adds 0.2.
    """
    lay = make_layer(1, 0)
    _, a = cla.pack(lay)
    n_w = lay.N * lay.K
    ideal = (3 * n_w + 8 * a["lut_or_scale"] + 8 * a["csr"]) / n_w
    assert abs(ideal - 3.24) < 0.02
    assert abs(8 * a["total"] / n_w - (ideal + 0.2)) < 0.01


def _bad(layer, status):
    with pytest.raises(cla.ClError) as e:
        cla.pack(layer)
    assert e.value.status == status, str(e.value)


def test_validation_errors():
    r = np.random.default_rng(4)
    base = make_layer(1, 0, K=50, N=10)
    base = base.with_(**dict(zip(("csr_row_ptr", "csr_col", "csr_val"), draw_csr(r, r, 10, 50, density=0.2))))
    c = base.codes.copy(); c[3, 7] = 8
    _bad(base.with_(codes=c), -1)                                   # code out of range
    col = base.csr_col.copy()
    rp = base.csr_row_ptr
    n = int(np.argmax(np.diff(rp) >= 2))
    col[rp[n]], col[rp[n] + 1] = col[rp[n] + 1], col[rp[n]]
    _bad(base.with_(csr_col=col), -1)                               # unsorted columns
    col2 = base.csr_col.copy(); col2[0] = 50
    _bad(base.with_(csr_col=col2), -1)                              # column out of range
    rp2 = base.csr_row_ptr.copy(); rp2[-1] += 1
    _bad(base.with_(csr_row_ptr=rp2), -1)                           # row_ptr[N] != nnz
    _bad(base.with_(mask="2:4", keep=np.ones((10, 50), np.uint8)), -2)  # mask on a LUT
    lay3 = make_layer(3, 0, K=64, N=8)
    keep = lay3.keep.copy(); keep[0, :4] = [1, 1, 1, 0]
    _bad(lay3.with_(keep=keep), -1)                                 # 2:4 group keeps three
    _bad(lay3.with_(K=62, qvals=lay3.qvals[:, :62], keep=lay3.keep[:, :62], L=lay3.L[:62]), -2)
    q = lay3.qvals.copy(); q[0, np.flatnonzero(lay3.keep[0])[0]] = 8
    _bad(lay3.with_(qvals=q), -1)                                   # int4 value out of range
    _bad(base.with_(K=0, codes=base.codes[:, :0]), -1)
    _bad(base.with_(act_clamp=np.float16(-1.0)), -1)
    f = np.full(3, 0.5, np.float16)
    _bad(base.with_(xscale_ch=np.array([1, 1, 4], np.int32), xscale=f), -1)      # repeated channel
    _bad(base.with_(xscale_ch=np.array([4, 1, 7], np.int32), xscale=f), -1)      # not increasing
    _bad(base.with_(xscale_ch=np.array([1, 4, 50], np.int32), xscale=f), -1)     # channel out of range
    for bad in (0.0, -0.5, 2.0, 2.0 ** -15, np.inf):                               # factor not normal in [2^-14, 1]
        _bad(base.with_(xscale_ch=np.array([1, 4, 7], np.int32), xscale=np.array([0.5, bad, 0.5], np.float16)), -1)
    cla.pack(base.with_(xscale_ch=np.array([1, 4, 49], np.int32), xscale=np.array([1.0, 2.0 ** -14, 0.75], np.float16)))


def test_size_query_and_small_buffer():
    import ctypes
    lay = make_layer(1, 0, K=40, N=3)
    keep = []
    d = cla._desc(lay, keep)
    size = ctypes.c_size_t(0)
    assert cla.lib().cl_pack(ctypes.byref(d), None, ctypes.byref(size), None) == 0
    buf = np.zeros(size.value, np.uint8)
    small = ctypes.c_size_t(size.value - 1)
    assert cla.lib().cl_pack(ctypes.byref(d), buf.ctypes.data, ctypes.byref(small), None) == -3
    assert small.value == size.value


def test_skewed_csr_roundtrip():
    r = np.random.default_rng(9)
    rp, col, val = draw_csr_skewed(r, r, 300, 700)
    lay = make_layer(1, 0, K=700, N=300).with_(csr_row_ptr=rp, csr_col=col, csr_val=val)
    _roundtrip(lay)
