"""Pins of the packer oracle (oracle/fit_oracle.py) against facts that do not
come from it: hand-derived examples, brute force, the fixed-point property of
Lloyd's iterations, scikit-learn's k-means and numpy's fp16 cast.  Each pin
takes the oracle module as an argument so that the mutation tests can run
them against broken copies."""
from __future__ import annotations

import numpy as np


def _rng(s):
    return np.random.default_rng(s)


def pin_worked_example(F):
    # SqueezeLLM page, Approach (per-channel centroids; outliers to CSR).
    # Row 0: 0..7 and 100.  100 is the one outlier; the dense values start from
    # c_j = 7 (2j + 1) / 16 = 0.4375, 1.3125, ..., 6.5625 with midpoints
    # 0.875, 1.75, ..., 6.125, so value j joins cluster j and c_j = j: LUT 0..7,
    # codes = values, the outlier takes the code nearest to 0 (code 0, value 0)
    # and its CSR value is 100 - 0 = 100.
    # Row 1: -4, -4, 0, 4, 4 x2: k = 8 from [-4, 4]: c_j = -4 + 8 (2j+1) / 16 =
    # -3.5, -2.5, ..., 3.5; -4 -> 0, 0 sits on the midpoint of c_3 = -0.5 and
    # c_4 = 0.5 -> cluster 3 (lower); 4 -> 7.  Means: c_0 = -4, c_3 = 0, c_7 = 4,
    # the others keep their values; next round: same assignment, stop.
    W = np.array([[0, 1, 2, 3, 4, 5, 6, 7, 100],
                  [-4, -4, 0, 4, 4, 4, 4, 4, 4]], np.float16)
    codes, lut, rp, col, val = F.fit_lut(W, 3, 1, 50)
    assert np.array_equal(lut[0].astype(np.float64), np.arange(8.0)), lut[0]
    assert np.array_equal(codes[0], [0, 1, 2, 3, 4, 5, 6, 7, 0])
    assert list(rp) == [0, 1, 1] and list(col) == [8] and float(val[0]) == 100.0
    assert np.array_equal(lut[1].astype(np.float64), [-4, -2.5, -1.5, 0, 0.5, 1.5, 2.5, 4])
    assert np.array_equal(codes[1], [0, 0, 3, 7, 7, 7, 7, 7, 7])


def pin_round_f16_library(F):
    r = _rng(61)
    v = r.normal(0, 1, 5000) * np.exp2(r.integers(-26, 14, 5000))
    h = r.integers(1, 0x7BFE, 3000).astype(np.uint16)
    mid = (h.view(np.float16).astype(np.float64) + (h + 1).view(np.float16).astype(np.float64)) / 2
    for x in (v, mid, -mid):
        assert np.array_equal(F.round_to_f16(x), x.astype(np.float16).astype(np.float64))


def pin_outliers_brute(F):
    r = _rng(62)
    W = r.normal(0, 1, (7, 13)).astype(np.float16)
    W[2, 3] = W[5, 1] = W[0, 12] = np.float16(-9.0)   # equal magnitudes: row-major order decides
    W[4, 4] = np.float16(9.0)
    for n_out in (0, 1, 3, 4, 5, 20, 91):
        m = F.select_outliers(W, n_out)
        flat = [(-abs(float(W.flat[i])), i) for i in range(W.size)]
        want = {i for _, i in sorted(flat)[:n_out]}
        assert set(np.flatnonzero(m.ravel())) == want, n_out
    m = F.select_outliers(W, 3)
    assert set(np.flatnonzero(m.ravel())) == {12, 3 + 13 * 2, 4 + 13 * 4}  # the three |w| = 9 of lowest index


def _assign(v, c):
    d = np.abs(v[:, None] - c[None, :])
    return np.argmin(d, axis=1)  # first (lower) index on a tie


def pin_kmeans_fixed_point(F):
    r = _rng(63)
    for k in (8, 16):
        for K in (5, 40, 333):
            v = (r.normal(0, 0.02, K) * (1 + 20 * (r.random(K) < 0.01))).astype(np.float16)
            v[: K // 5] = v[K // 5: 2 * (K // 5)]             # duplicates
            c = F.kmeans_row(v, k, 500)
            x = v.astype(np.float64)
            lab = _assign(x, c)
            for j in range(k):
                if (lab == j).any():
                    assert abs(c[j] - x[lab == j].mean()) <= 1e-12 * max(1e-300, abs(c[j])) + 1e-18, (k, K, j)
            # nearest-centroid assignment is what the boundaries give
            b = (c[:-1] + c[1:]) * 0.5
            assert np.array_equal(np.searchsorted(b, x, side="left"), lab)


def pin_kmeans_sklearn(F):
    from sklearn.cluster import KMeans
    r = _rng(64)
    checked = 0
    for t in range(12):
        k = 8
        v = r.normal(0, 0.02, 400).astype(np.float16)
        x = v.astype(np.float64)
        init = x.min() + ((x.max() - x.min()) * (2 * np.arange(k) + 1)) / (2 * k)
        c = F.kmeans_row(v, k, 300)
        km = KMeans(n_clusters=k, init=init.reshape(-1, 1), n_init=1, max_iter=300, tol=0.0,
                    algorithm="lloyd").fit(x.reshape(-1, 1))
        lab = _assign(x, c)
        if len(set(lab)) < k:
            continue  # an empty cluster: scikit-learn relocates it, the page's reading keeps it
        assert np.allclose(np.sort(km.cluster_centers_.ravel()), c, rtol=0, atol=1e-12)
        checked += 1
    assert checked >= 6


def pin_sse_monotone(F):
    r = _rng(65)
    v = r.standard_t(3, 700).astype(np.float16) * np.float16(0.01)
    x = v.astype(np.float64)
    prev = np.inf
    for it in range(1, 15):
        c = F.kmeans_row(v, 16, it)
        sse = float(((x - c[_assign(x, c)]) ** 2).sum())
        assert sse <= prev * (1 + 1e-12)
        prev = sse


def pin_codes_and_residual(F):
    r = _rng(66)
    W = (r.normal(0, 0.02, (9, 150)) * (1 + 40 * (r.random((9, 150)) < 0.005))).astype(np.float16)
    for bits in (3, 4):
        codes, lut, rp, col, val = F.fit_lut(W, bits, 14, 60)
        out = np.zeros(W.shape, bool)
        for n in range(9):
            out[n, col[rp[n]:rp[n + 1]]] = True
        assert out.sum() == 14
        assert np.all(np.diff(lut.astype(np.float64), axis=1) >= 0)
        w = W.astype(np.float64)
        l = lut.astype(np.float64)
        for n in range(9):
            tgt = np.where(out[n], 0.0, w[n])
            assert np.array_equal(codes[n], np.argmin(np.abs(tgt[:, None] - l[n][None, :]), axis=1))
            for p in range(rp[n], rp[n + 1]):
                j = col[p]
                exact = w[n, j] - l[n, codes[n, j]]
                assert float(val[p]) == float(np.float16(exact))
        # outliers are the largest magnitudes
        assert np.abs(w[out]).min() >= np.abs(w[~out]).max()


# ---------------------------------------------------------------------------
# integer formats: masks and the clip search
# ---------------------------------------------------------------------------

def pin_int_worked_example(F):
    # SLiM page, highlights (symmetric quantization, clipping, grid search).
    # w = [1, -2, 3, 0.5, 0.25, -7, 6, 0], qmax = 7, G = 4: m = 7, s_i = i/4.
    #   s = 1:    q = [1,-2,3,0,0,-7,6,0] (0.5 rounds to even 0); err = 0.5^2 + 0.25^2 = 0.3125
    #   s = 0.75: q = [1,-3,4,1,0,-7,7,0]; err = 4 * 0.0625 + 1.75^2 + 0.75^2 = 3.875
    #   s = 0.5:  q = [2,-4,6,1,0,-7,7,0]; err = 0.0625 + 3.5^2 + 2.5^2 = 18.5625
    #   s = 0.25: larger still.  Best: s = 1.
    w = np.array([[1, -2, 3, 0.5, 0.25, -7, 6, 0]], np.float16)
    q, s, keep = F.fit_int(w, 4, "none", 4)
    assert float(s[0]) == 1.0 and list(q[0]) == [1, -2, 3, 0, 0, -7, 6, 0]
    # 2:4 keeps (-2, 3) and (-7, 6): all on the grid at s = 1, error 0
    q, s, keep = F.fit_int(w, 4, "2:4", 4)
    assert list(keep[0]) == [0, 1, 1, 0, 0, 1, 1, 0] and float(s[0]) == 1.0
    assert list(q[0]) == [0, -2, 3, 0, 0, -7, 6, 0]


def _beaten(a, i, idx):
    return sum(1 for u in idx if a[u] > a[i] or (a[u] == a[i] and u < i))


def pin_masks_brute(F):
    r = _rng(71)
    W = r.choice(np.array([-1.0, -0.5, 0.5, 1.0, 2.0, 0.0], np.float16), size=(6, 24))  # many ties
    a = np.abs(W.astype(np.float64))
    k24 = F.magnitude_mask(W, "2:4")
    kh = F.magnitude_mask(W, "half")
    for n in range(6):
        for t in range(24):
            g = list(range(4 * (t // 4), 4 * (t // 4) + 4))
            assert k24[n, t] == (1 if _beaten(a[n], t, g) < 2 else 0)
            assert kh[n, t] == (1 if _beaten(a[n], t, range(24)) < 12 else 0)
    assert np.all(k24.reshape(6, 6, 4).sum(axis=2) == 2) and np.all(kh.sum(axis=1) == 12)


def pin_clip_search_fractions(F):
    # exact errors with Fractions, an independent route to the same argmin
    from fractions import Fraction
    r = _rng(72)
    for bits, G in ((4, 12), (8, 6)):
        qmax = (1 << (bits - 1)) - 1
        for t in range(6):
            w = (r.normal(0, 0.02, 40) * (1 + 8 * (r.random(40) < 0.05))).astype(np.float16)
            kept = r.random(40) < 0.7
            s, q = F.clip_search_row(w, kept, bits, G)
            m = max(abs(Fraction(float(v))) for v in w[kept])
            best = None
            for i in range(1, G + 1):
                si = float(np.float16(float(Fraction(i) * m / (qmax * G))))
                if si == 0:
                    continue
                qi = [max(-qmax, min(qmax, int(np.rint(float(v) / si)))) for v in w[kept]]
                err = sum((Fraction(float(v)) - Fraction(si) * b) ** 2 for v, b in zip(w[kept], qi))
                if best is None or err < best[0]:
                    best = (err, si, qi)
            assert float(s) == best[1]
            assert list(q[kept]) == best[2] and not q[~kept].any()


def pin_clip_never_worse_than_absmax(F):
    r = _rng(73)
    W = (r.standard_t(3, (5, 64)) * 0.01).astype(np.float16)
    q, s, keep = F.fit_int(W, 4, "none", 20)
    w = W.astype(np.float64)
    for n in range(5):
        err = ((w[n] - float(s[n]) * q[n]) ** 2).sum()
        s1 = float(np.float16(np.abs(w[n]).max() / 7))
        q1 = np.clip(np.rint(w[n] / s1), -7, 7)
        assert err <= ((w[n] - s1 * q1) ** 2).sum() * (1 + 1e-12)
        assert np.abs(q[n]).max() <= 7


# ---------------------------------------------------------------------------
# AbsMax group quantization of factors
# ---------------------------------------------------------------------------

def pin_absmax_worked_example(F):
    # SLiM page, highlights (AbsMax groups).  Column 0, group 4: [0.875, -1.75, 0.375, 0]:
    # max = 1.75, scale = 1.75 / 7 = 0.25 (exact); v / s = [3.5, -7, 1.5, 0] -> rint (ties to
    # even) [4, -7, 2, 0].  Ragged second group [0.4375]: scale 0.0625, q = 7.
    # Column 1 is all zero: scale 0, q 0.
    v = np.array([[0.875, 0], [-1.75, 0], [0.375, 0], [0, 0], [0.4375, 0]], np.float16)
    q, sc = F.absmax_groups(v, 4)
    assert float(sc[0, 0]) == 0.25 and float(sc[0, 1]) == 0.0 and float(sc[1, 0]) == 0.0625
    assert list(q[:, 0]) == [4, -7, 2, 0, 7] and not q[:, 1].any()


def pin_absmax_properties(F):
    r = _rng(74)
    for dtype in ("f16", "bf16"):
        for R, C, g in ((300, 5, 128), (37, 3, 8), (10, 4, 1)):
            x = r.normal(0, 0.01, (R, C))
            if dtype == "bf16":
                v = (np.ascontiguousarray(x.astype(np.float32)).view(np.uint32) + 0x8000 >> 16).astype(np.uint16)
                vf = (v.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
            else:
                v = x.astype(np.float16)
                vf = v.astype(np.float64)
            q, sc = F.absmax_groups(v, g, dtype)
            assert sc.shape == (-(-R // g), C) and np.abs(q).max() <= 7
            s_full = np.repeat(sc.astype(np.float64), g, axis=0)[:R]
            # every value is within half a step of its code, and each group's
            # largest magnitude maps to +-7
            assert np.all(np.abs(vf - s_full * q) <= s_full / 2 + 1e-300)
            for gi in range(sc.shape[0]):
                blk = np.abs(vf[gi * g:(gi + 1) * g])
                for c in range(C):
                    j = int(np.argmax(blk[:, c]))
                    assert abs(int(q[gi * g + j, c])) == 7


def pin_lora_worked_examples(F):
    # SLiM page, review highlights, SLiM-LoRA bullet (Naive-LoRA: least error norm).
    # diag(3, 1, 2): the best rank-2 approximation keeps 3 and 2 and drops 1.
    E = np.diag([3.0, 1.0, 2.0])
    L, R, s = F.naive_lora(E, 2)
    assert np.allclose((L @ R).T, np.diag([3.0, 0.0, 2.0]), atol=1e-12), (L @ R).T
    assert np.allclose(s, [3.0, 2.0])
    # a rank-1 matrix a b^T: one factor pair reproduces it, sigma = |a| |b| = 5 * 13
    a, b = np.array([3.0, 4.0]), np.array([5.0, 0.0, 12.0])
    L, R, s = F.naive_lora(np.outer(a, b), 1)
    assert np.allclose((L @ R).T, np.outer(a, b), atol=1e-12) and abs(s[0] - 65.0) < 1e-12
    # the square-root split: L^T L = R R^T = diag(s)
    assert np.allclose(L.T @ L, np.diag(s)) and np.allclose(R @ R.T, np.diag(s))
    # rank past min(N, K): exact, zero columns beyond
    L, R, s = F.naive_lora(np.outer(a, b), 4)
    assert np.allclose((L @ R).T, np.outer(a, b), atol=1e-12) and np.all(L[:, 2:] == 0) and np.all(s[2:] == 0)


def pin_lora_eckart_young(F):
    # the error of the truncation is the root-sum-square of the dropped singular
    # values, here from the eigenvalues of E^T E (another routine); no rank-r
    # matrix does better than it (random rank-r candidates, and the best one
    # perturbed); the factors' product does not depend on SVD sign choices
    # (E and -E, E and E^T give the negated / transposed products)
    r = _rng(77)
    for N, K, rank in ((40, 25, 5), (17, 60, 3), (30, 30, 29)):
        E = r.normal(0, 1, (N, K)) * np.exp(-np.arange(K) / 9.0)
        L, R, s = F.naive_lora(E, rank)
        A = (L @ R).T
        lam = np.sort(np.linalg.eigvalsh(E.T @ E))[::-1]
        err = np.linalg.norm(E - A)
        assert abs(err - np.sqrt(max(lam[rank:].sum(), 0.0))) <= 1e-9 * np.linalg.norm(E), (err, lam[rank:].sum())
        assert np.allclose(s ** 2, lam[:rank], rtol=1e-9, atol=1e-9 * lam[0])
        for _ in range(5):
            B = r.normal(0, 1, (N, rank)) @ r.normal(0, 1, (rank, K))
            B *= np.vdot(B, E) / np.vdot(B, B)  # the best multiple of a random rank-r matrix
            assert np.linalg.norm(E - B) >= err
            P = ((L + 1e-3 * r.normal(0, 1, L.shape)) @ (R + 1e-3 * r.normal(0, 1, R.shape))).T  # rank r still
            assert np.linalg.norm(E - P) >= err - 1e-12
        L2, R2, _ = F.naive_lora(-E, rank)
        assert np.allclose((L2 @ R2).T, -A, atol=1e-9)
        L3, R3, _ = F.naive_lora(E.T, rank)
        assert np.allclose(L3 @ R3, A, atol=1e-9)


ALL_PINS = [pin_worked_example, pin_round_f16_library, pin_outliers_brute, pin_kmeans_fixed_point,
            pin_kmeans_sklearn, pin_sse_monotone, pin_codes_and_residual, pin_int_worked_example,
            pin_masks_brute, pin_clip_search_fractions, pin_clip_never_worse_than_absmax,
            pin_absmax_worked_example, pin_absmax_properties, pin_lora_worked_examples, pin_lora_eckart_young]


def failing_pins(F):
    bad = []
    for p in ALL_PINS:
        try:
            p(F)
        except Exception as e:  # noqa: BLE001
            bad.append((p.__name__, repr(e)[:200]))
    return bad
