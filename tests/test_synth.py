"""The seeded generator produces the workloads' shapes, distributions and structure (no GPU)."""
import numpy as np
import pytest

from synth.layers import CONFIGS, make_layer, make_x, f32_from_bf16_bits, bf16_bits_from_f32


def test_reproducible():
    a = make_layer(1, 0, K=200, N=70)
    b = make_layer(1, 0, K=200, N=70)
    assert np.array_equal(a.codes, b.codes) and np.array_equal(a.csr_col, b.csr_col)
    assert np.array_equal(make_x(1, 0, 2, K=200), make_x(1, 0, 2, K=200))


@pytest.mark.parametrize("cfg", [1, 2, 5])
def test_lut_layers(cfg):
    lay = make_layer(cfg, 0, K=1000, N=300)
    bits = 3 if cfg != 2 else 4
    assert lay.dense == f"lut{bits}" and lay.codes.max() < (1 << bits)
    assert lay.lut.shape == (300, 1 << bits) and lay.lut.dtype == np.float16
    assert (np.diff(lay.lut.astype(np.float64), axis=1) >= 0).all()          # sorted
    assert lay.nnz == round(0.0045 * 300 * 1000)
    rp, col = lay.csr_row_ptr, lay.csr_col
    for n in range(lay.N):
        c = col[rp[n]:rp[n + 1]]
        assert (np.diff(c) > 0).all() and (c < lay.K).all()
    if cfg == 5:
        assert lay.lr == "bf16" and lay.rank == 64 and lay.L.shape == (1000, 64) and lay.R.shape == (64, 300)


def test_cfg3_int4_2_4():
    lay = make_layer(3, 0, K=512, N=96)
    keep = lay.keep.reshape(96, 128, 4)
    assert (keep.sum(axis=2) == 2).all()
    assert lay.qvals.min() >= -8 and lay.qvals.max() <= 7
    assert (lay.row_scale.view(np.uint16) == 0x19DA).all()
    assert lay.L_scale.shape == (4, 128) and lay.R_scale.shape == (1, 96)
    x = make_x(3, 0, 8, K=512)
    big = np.abs(x.astype(np.float64)).max(axis=0) > 8
    assert 0 < big.sum() <= round(0.001 * 512) + 1


def test_cfg4_int8_bitmap_clamp():
    lay = make_layer(4, 0, K=640, N=64)
    assert (lay.keep.sum(axis=1) == 320).all()
    assert np.abs(lay.qvals.astype(np.int32)).max() == 127
    assert lay.act_clamp is not None and float(lay.act_clamp) > 3.0


def test_bf16_rounding():
    v = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 1e-40], np.float32)
    b = bf16_bits_from_f32(v)
    assert b.tolist() == [0x3F80, 0x3F80, 0x3F82, 0xC020, 0x0001] or b[:4].tolist() == [0x3F80, 0x3F80, 0x3F82, 0xC020]
    assert np.array_equal(f32_from_bf16_bits(np.array([0x3F80, 0xC020], np.uint16)), np.array([1.0, -2.5], np.float32))


def test_configs_table():
    assert [len(CONFIGS[c]["layers"]) for c in range(1, 6)] == [1, 5, 2, 2, 3]
