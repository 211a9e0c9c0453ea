"""The packer oracle against its pins, and planted mistakes in copies of it (no GPU)."""
import importlib.util
import os

import numpy as np
import pytest

import fit_pins

FIT_FILE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "fit_oracle.py")


def fresh():
    spec = importlib.util.spec_from_file_location("fit_mutant", FIT_FILE)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.parametrize("pin", fit_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_fit_pin(pin):
    pin(fresh())


def _mut_outliers_signed(F):
    def select_outliers(W, n_out):
        a = np.asarray(W, np.float16).astype(np.float64).ravel()
        order = np.lexsort((np.arange(a.size), -a))
        m = np.zeros(a.size, bool)
        m[order[:n_out]] = True
        return m.reshape(np.asarray(W).shape)
    F.select_outliers = select_outliers


def _mut_outlier_ties_high(F):
    def select_outliers(W, n_out):
        a = np.abs(np.asarray(W, np.float16).astype(np.float64)).ravel()
        order = np.lexsort((-np.arange(a.size), -a))
        m = np.zeros(a.size, bool)
        m[order[:n_out]] = True
        return m.reshape(np.asarray(W).shape)
    F.select_outliers = select_outliers


def _kmeans_variant(F, init="even", side="left", empty="keep", one_pass=False):
    def kmeans_row(v16, k, max_iter):
        v = np.asarray(v16, np.float16).astype(np.float64)
        if v.size == 0:
            return np.zeros(k)
        mn, mx = v.min(), v.max()
        c = mn + (mx - mn) * np.arange(k) / (k - 1) if init == "ends" else mn + ((mx - mn) * (2 * np.arange(k) + 1)) / (2 * k)
        for _ in range(1 if one_pass else max_iter):
            b = (c[:-1] + c[1:]) * 0.5
            idx = np.searchsorted(b, v, side=side)
            sums = np.zeros(k)
            np.add.at(sums, idx, v)
            cnt = np.bincount(idx, minlength=k)
            new = c.copy() if empty == "keep" else np.zeros(k)
            nz = cnt > 0
            new[nz] = sums[nz] / cnt[nz]
            if np.array_equal(new, c):
                break
            c = new
        return c
    F.kmeans_row = kmeans_row


def _mut_init_ends(F):
    _kmeans_variant(F, init="ends")


def _mut_ties_upper(F):
    _kmeans_variant(F, side="right")


def _mut_empty_to_zero(F):
    _kmeans_variant(F, empty="zero")


def _mut_one_iteration(F):
    _kmeans_variant(F, one_pass=True)


def _mut_lut_truncated(F):
    orig = F.round_to_f16

    def round_to_f16(v):
        v = np.asarray(v, np.float64)
        r = orig(v)
        _, e = np.frexp(v)
        sp = np.ldexp(1.0, np.maximum(e - 1, -14) - 10)
        return np.where(np.abs(r) > np.abs(v), r - np.sign(v) * sp, r)
    F.round_to_f16 = round_to_f16


def _mut_code_ties_upper(F):
    def nearest_code(v, lut16):
        l = np.asarray(lut16, np.float16).astype(np.float64)
        b = (l[:-1] + l[1:]) * 0.5
        return np.searchsorted(b, np.asarray(v, np.float64), side="right").astype(np.uint8)
    F.nearest_code = nearest_code


def _mut_outlier_code_nearest_w(F):
    orig_fit = F.fit_lut

    def fit_lut(W, bits, n_out, max_iter):
        codes, lut, rp, col, val = orig_fit(W, bits, n_out, max_iter)
        W16 = np.asarray(W, np.float16)
        for n in range(W16.shape[0]):
            for p in range(rp[n], rp[n + 1]):
                j = col[p]
                codes[n, j] = F.nearest_code(np.array([float(W16[n, j])]), lut[n])[0]
                val[p] = np.float16(float(W16[n, j]) - float(lut[n, codes[n, j]]))
        return codes, lut, rp, col, val
    F.fit_lut = fit_lut


MUTANTS = [_mut_outliers_signed, _mut_outlier_ties_high, _mut_init_ends, _mut_ties_upper, _mut_empty_to_zero,
           _mut_one_iteration, _mut_lut_truncated, _mut_code_ties_upper, _mut_outlier_code_nearest_w]


@pytest.mark.parametrize("mutate", MUTANTS, ids=lambda f: f.__name__[5:])
def test_fit_pins_catch_mutant(mutate):
    F = fresh()
    mutate(F)
    assert fit_pins.failing_pins(F), f"no pin caught {mutate.__name__}"


def _mut_mask_ties_high(F):
    orig = F.magnitude_mask

    def magnitude_mask(W, kind):
        W = np.asarray(W, np.float16)
        return orig(W[:, ::-1], kind)[:, ::-1] if kind != "2:4" else \
            orig(W.reshape(W.shape[0], -1, 4)[:, :, ::-1].reshape(W.shape), kind).reshape(W.shape[0], -1, 4)[:, :, ::-1].reshape(W.shape)
    F.magnitude_mask = magnitude_mask


def _mut_mask_signed(F):
    orig = F.magnitude_mask

    def magnitude_mask(W, kind):
        W = np.asarray(W, np.float16)
        shifted = (W.astype(np.float64) + 100.0).astype(np.float16)  # ranks by signed value
        return orig(shifted, kind)
    F.magnitude_mask = magnitude_mask


def _clip_variant(F, qmax_plus=0, err_all=False, worst=False, trunc=False):
    def clip_search_row(w16, kept, bits, grid):
        qmax = (1 << (bits - 1)) - 1 + qmax_plus
        w = np.asarray(w16, np.float16).astype(np.float64)
        k = np.asarray(kept, bool)
        q = np.zeros(w.size, np.int64)
        m = float(np.abs(w[k]).max()) if k.any() else 0.0
        best = None
        for i in range(1, grid + 1):
            s = float(F.round_to_f16((i * m) / ((qmax - qmax_plus) * grid)))
            if s == 0.0:
                continue
            rnd = np.trunc if trunc else np.rint
            qi = np.clip(rnd(w[k] / s), -qmax, qmax).astype(np.int64)
            err = ((w[k] - s * qi) ** 2).sum() + (((w[~k]) ** 2).sum() if err_all else 0.0)
            better = best is None or (err > best[0] if worst else err < best[0])
            if better:
                best = (err, s, qi)
        if best is None:
            return np.float16(0.0), q.astype(np.int8)
        q[k] = best[2]
        return np.float16(best[1]), q.astype(np.int8)
    F.clip_search_row = clip_search_row


def _mut_qmax_asymmetric(F):
    _clip_variant(F, qmax_plus=1)


def _mut_worst_scale(F):
    _clip_variant(F, worst=True)


def _mut_truncating_codes(F):
    _clip_variant(F, trunc=True)


INT_MUTANTS = [_mut_mask_ties_high, _mut_mask_signed, _mut_qmax_asymmetric, _mut_worst_scale, _mut_truncating_codes]


@pytest.mark.parametrize("mutate", INT_MUTANTS, ids=lambda f: f.__name__[5:])
def test_fit_pins_catch_int_mutant(mutate):
    F = fresh()
    mutate(F)
    assert fit_pins.failing_pins(F), f"no pin caught {mutate.__name__}"


def _mut_absmax_axis(F):
    orig = F.absmax_groups

    def absmax_groups(F16, group, dtype="f16"):
        q, sc = orig(np.asarray(F16).T, group, dtype)
        ng = -(-np.asarray(F16).shape[0] // group)
        return q.T, np.resize(sc.T, (ng, np.asarray(F16).shape[1])).astype(np.float16)
    F.absmax_groups = absmax_groups


def _mut_absmax_div8(F):
    src = F.absmax_groups

    def absmax_groups(F16, group, dtype="f16"):
        q, sc = src(F16, group, dtype)
        return np.clip(np.rint(q * 7 / 8), -8, 7).astype(np.int8), (sc.astype(np.float64) * 8 / 7).astype(np.float16)
    F.absmax_groups = absmax_groups


@pytest.mark.parametrize("mutate", [_mut_absmax_axis, _mut_absmax_div8], ids=lambda f: f.__name__[5:])
def test_fit_pins_catch_absmax_mutant(mutate):
    F = fresh()
    mutate(F)
    assert fit_pins.failing_pins(F), f"no pin caught {mutate.__name__}"


# Naive-LoRA: planted mistakes the pins must catch
def _mut_lora_smallest(F):
    def naive_lora(E, rank):
        E = np.asarray(E, dtype=np.float64)
        U, s, Vt = np.linalg.svd(E, full_matrices=False)
        idx = np.argsort(s)[:rank]  # the smallest singular values instead of the largest
        sq = np.sqrt(s[idx])
        return Vt[idx].T * sq, (U[:, idx] * sq).T, s[idx]
    F.naive_lora = naive_lora


def _mut_lora_unsplit(F):
    def naive_lora(E, rank):
        E = np.asarray(E, dtype=np.float64)
        U, s, Vt = np.linalg.svd(E, full_matrices=False)
        r = min(rank, s.size)
        L = np.zeros((E.shape[1], rank)); R = np.zeros((rank, E.shape[0])); sv = np.zeros(rank)
        L[:, :r] = Vt[:r].T * s[:r]  # all of s in L
        R[:r] = U[:, :r].T
        sv[:r] = s[:r]
        return L, R, sv
    F.naive_lora = naive_lora


def _mut_lora_transposed(F):
    def naive_lora(E, rank):
        E = np.asarray(E, dtype=np.float64)
        U, s, Vt = np.linalg.svd(E, full_matrices=False)
        r = min(rank, s.size)
        sq = np.sqrt(s[:r])
        L = np.zeros((E.shape[1], rank)); R = np.zeros((rank, E.shape[0])); sv = np.zeros(rank)
        L[:, :r] = (U[:, :r] * sq)[:E.shape[1]] if E.shape[0] >= E.shape[1] else np.pad(U[:, :r] * sq, ((0, E.shape[1] - E.shape[0]), (0, 0)))
        R[:r] = (Vt[:r].T * sq).T[:, :E.shape[0]] if E.shape[1] >= E.shape[0] else np.pad((Vt[:r].T * sq).T, ((0, 0), (0, E.shape[0] - E.shape[1])))
        sv[:r] = s[:r]
        return L, R, sv
    F.naive_lora = naive_lora


LORA_MUTANTS = [_mut_lora_smallest, _mut_lora_unsplit, _mut_lora_transposed]


@pytest.mark.parametrize("mutate", LORA_MUTANTS, ids=lambda f: f.__name__[5:])
def test_lora_mutant_caught(mutate):
    F = fresh()
    mutate(F)
    assert fit_pins.failing_pins(F), "no pin caught the planted mistake"
