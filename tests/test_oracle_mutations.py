"""Plant plausible mistakes in copies of the CPU oracle and check that the pins catch each one.

Every mutant is a fresh copy of the oracle module with one function replaced
on the CPU; the real oracle is never modified.
"""
import importlib.util
import os

import numpy as np
import pytest

import oracle_pins

ORACLE_FILE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                           "oracle", "compressed_linear_oracle.py")


def fresh_oracle():
    spec = importlib.util.spec_from_file_location("oracle_mutant", ORACLE_FILE)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _mut_mask_ignored(O):
    orig = O.dense_plane

    def dense_plane(layer, rows=None):
        return orig(layer.with_(mask="none"), rows)
    O.dense_plane = dense_plane


def _mut_scale_per_column(O):
    def dense_plane(layer, rows=None):
        idx = O._rows(layer, rows)
        if layer.dense.startswith("int"):
            q = layer.qvals[idx].astype(np.float64)
            s = layer.row_scale.astype(np.float64)
            cols = np.arange(layer.K) % s.size
            D = q * s[cols][None, :]
            if layer.mask != "none":
                D = np.where(layer.keep[idx].astype(bool), D, 0.0)
            return D
        lut = layer.lut.astype(np.float64)[idx]
        return np.take_along_axis(lut, layer.codes[idx].astype(np.int64), axis=1)
    O.dense_plane = dense_plane


def _mut_lut_off_by_one(O):
    orig = O.dense_plane

    def dense_plane(layer, rows=None):
        if layer.dense.startswith("lut"):
            nb = layer.lut.shape[1]
            return orig(layer.with_(codes=((layer.codes.astype(np.int64) + 1) % nb).astype(np.uint8)), rows)
        return orig(layer, rows)
    O.dense_plane = dense_plane


def _mut_sparse_dropped(O):
    O.sparse_plane = lambda layer, rows=None: np.zeros((O._rows(layer, rows).size, layer.K))


def _mut_sparse_sign(O):
    orig = O.sparse_plane
    O.sparse_plane = lambda layer, rows=None: -orig(layer, rows)


def _mut_sparse_col_shift(O):
    orig = O.sparse_plane
    O.sparse_plane = lambda layer, rows=None: np.roll(orig(layer, rows), 1, axis=1)


def _mut_lowrank_dropped(O):
    O.lowrank_factors = lambda layer: (None, None)


def _mut_lowrank_group_axis(O):
    def _dequant_groups(q, scale, group):
        qf = np.asarray(q).astype(np.float64)
        sf = np.asarray(scale, dtype=np.float16).astype(np.float64)
        cols = np.arange(qf.shape[1]) // group
        return qf * sf[0][None, :] if sf.shape[0] else qf
    O._dequant_groups = _dequant_groups


def _mut_lowrank_R_transposed_use(O):
    orig = O.lowrank_factors

    def lowrank_factors(layer):
        Lh, Rh = orig(layer)
        if Lh is None:
            return Lh, Rh
        return Lh, Rh[::-1]  # rank index reversed
    O.lowrank_factors = lowrank_factors


def _mut_clamp_missing(O):
    orig = O.activations
    O.activations = lambda layer, x: orig(layer.with_(act_clamp=None), x)


def _mut_clamp_one_sided(O):
    def activations(layer, x):
        xf = O._act_to_f64(x, layer.x_dtype)
        if xf.ndim == 1:
            xf = xf[None, :]
        if layer.act_clamp is not None:
            xf = np.minimum(xf, float(layer.act_clamp))
        return xf
    O.activations = activations


def _mut_bf16_shift(O):
    O._bf16_to_f64 = lambda bits: (np.asarray(bits, np.uint16).astype(np.uint32) << np.uint32(15)).view(np.float32).astype(np.float64)


def _mut_forward_transposed(O):
    def forward(layer, x, rows=None):
        xp = O.activations(layer, x)
        W = O.reconstruct(layer, rows)
        y = xp @ W.T
        return y[:, ::-1]
    O.forward = forward


def _mut_debug_planes_truncate(O):
    orig = O.debug_planes

    def debug_planes(layer, rows=None):
        D16, S16, L32, R32 = orig(layer, rows)
        D = O.dense_plane(layer, rows)
        D16 = np.sign(D) * np.floor(np.abs(D) * 2 ** 16) / 2 ** 16  # truncation, not nearest
        return D16.astype(np.float16), S16, L32, R32
    O.debug_planes = debug_planes


def _scaled_activations(O, order="clamp_first", rnd=None, factor=lambda f: f, shift=0):
    """activations() with the channel scaling rebuilt with one planted change."""
    rnd = rnd or O.round_to_act

    def activations(layer, x):
        xf = O._act_to_f64(x, layer.x_dtype)
        if xf.ndim == 1:
            xf = xf[None, :]
        c = layer.act_clamp
        ch = layer.xscale_ch
        if ch is not None and len(ch) and order == "scale_first":
            f = factor(np.asarray(layer.xscale, np.float16).astype(np.float64))
            cols = (np.asarray(ch, np.int64) + shift) % layer.K
            xf = xf.copy()
            xf[:, cols] = rnd(xf[:, cols] * f[None, :], layer.x_dtype)
        if c is not None:
            xf = np.minimum(np.maximum(xf, -float(c)), float(c))
        if ch is not None and len(ch) and order == "clamp_first":
            f = factor(np.asarray(layer.xscale, np.float16).astype(np.float64))
            cols = (np.asarray(ch, np.int64) + shift) % layer.K
            xf = xf.copy()
            xf[:, cols] = rnd(xf[:, cols] * f[None, :], layer.x_dtype)
        return xf
    return activations


def _mut_xscale_ignored(O):
    orig = O.activations
    O.activations = lambda layer, x: orig(layer.with_(xscale_ch=None, xscale=None), x)


def _mut_xscale_times_alpha(O):
    O.activations = _scaled_activations(O, factor=lambda f: 1.0 / f)


def _mut_xscale_channel_shift(O):
    O.activations = _scaled_activations(O, shift=1)


def _mut_xscale_before_clamp(O):
    O.activations = _scaled_activations(O, order="scale_first")


def _mut_xscale_unrounded(O):
    O.activations = _scaled_activations(O, rnd=lambda v, dt: v)


def _mut_xscale_round_to_f16_always(O):
    O.activations = _scaled_activations(O, rnd=lambda v, dt: O.round_to_act(v, "f16"))


def _mut_round_truncate(O):
    orig = O.round_to_act

    def round_to_act(v, x_dtype):
        v = np.asarray(v, np.float64)
        r = orig(v, x_dtype)
        # toward zero: step back where nearest rounding went away from zero
        p, emin = O._ACT_FORMATS[x_dtype]
        _, e = np.frexp(v)
        sp = np.ldexp(1.0, np.maximum(e - 1, emin) - (p - 1))
        return np.where(np.abs(r) > np.abs(v), r - np.sign(v) * sp, r)
    O.round_to_act = round_to_act


def _mut_round_half_away(O):
    def round_to_act(v, x_dtype):
        p, emin = O._ACT_FORMATS[x_dtype]
        v = np.asarray(v, np.float64)
        _, e = np.frexp(v)
        sp = np.ldexp(1.0, np.maximum(e - 1, emin) - (p - 1))
        return np.sign(v) * np.floor(np.abs(v) / sp + 0.5) * sp
    O.round_to_act = round_to_act


def _mut_round_no_subnormals(O):
    def round_to_act(v, x_dtype):
        p, _ = O._ACT_FORMATS[x_dtype]
        v = np.asarray(v, np.float64)
        _, e = np.frexp(v)
        sp = np.ldexp(1.0, e - 1 - (p - 1))
        return np.rint(v / sp) * sp
    O.round_to_act = round_to_act


def _mut_fab_bound_signed(O):
    # forward_and_bound's tolerance taken on W_hat instead of |W_hat|
    def forward_and_bound(layer, x, rows=None):
        xp = O.activations(layer, x)
        W = O.reconstruct(layer, rows)
        return xp @ W.T, O.TOL_REL * np.abs(np.abs(xp) @ W.T)
    O.forward_and_bound = forward_and_bound


def _mut_fab_no_rank_term(O):
    # forward_and_bound's y built from D + S only
    def forward_and_bound(layer, x, rows=None):
        xp = O.activations(layer, x)
        idx = O._rows(layer, rows)
        W = O.reconstruct(layer, rows)
        Wds = O.dense_plane(layer, idx) + O.sparse_plane(layer, idx)
        return xp @ Wds.T, O.TOL_REL * (np.abs(xp) @ np.abs(W).T)
    O.forward_and_bound = forward_and_bound


MUTANTS = [
    _mut_mask_ignored, _mut_scale_per_column, _mut_lut_off_by_one, _mut_sparse_dropped,
    _mut_sparse_sign, _mut_sparse_col_shift, _mut_lowrank_dropped, _mut_lowrank_group_axis,
    _mut_lowrank_R_transposed_use, _mut_clamp_missing, _mut_clamp_one_sided, _mut_bf16_shift,
    _mut_forward_transposed, _mut_debug_planes_truncate,
    _mut_xscale_ignored, _mut_xscale_times_alpha, _mut_xscale_channel_shift, _mut_xscale_before_clamp,
    _mut_xscale_unrounded, _mut_xscale_round_to_f16_always, _mut_round_truncate, _mut_round_half_away,
    _mut_round_no_subnormals, _mut_fab_bound_signed, _mut_fab_no_rank_term,
]


def test_unmutated_copy_passes():
    assert oracle_pins.failing_pins(fresh_oracle()) == []


@pytest.mark.parametrize("mutate", MUTANTS, ids=lambda f: f.__name__[5:])
def test_pins_catch_mutant(mutate):
    O = fresh_oracle()
    mutate(O)
    assert oracle_pins.failing_pins(O), f"no pin caught {mutate.__name__}"
