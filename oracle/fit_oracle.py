"""CPU oracle of the data-free packers -- TEST INFRASTRUCTURE.

Only the test suite may import or run this module.  The HIP library never
calls it and it never calls the HIP library; they share no code.

What it computes, from fp16 weights W [N, K] (rows = output channels):

  1. Outliers.  The n_out weights of largest magnitude leave the dense part
     for a full-precision CSR matrix; among equal magnitudes the one with the
     smaller row-major index goes first.
  2. Per-row k-means.  The remaining weights of each row are clustered into
     2^b centroids by Lloyd's iterations in one dimension, starting from 2^b
     points spread evenly over [min, max] of the row:
         c_j = min + (max - min) (2j + 1) / 2^(b+1)
     A weight belongs to the nearest centroid (the lower one on a tie, i.e.
     to cluster j when it equals the midpoint of c_j and c_(j+1)); a centroid
     becomes the mean of its weights, and keeps its value when it has none.
     Iterations stop when no centroid changes, or after max_iter.
  3. Codes.  The LUT is the centroids rounded to fp16 (nearest, ties to even);
     every dense weight takes the code of its nearest LUT value (lower code on
     a tie).  An outlier's position takes the code nearest to 0 and its CSR
     value is fp16(w - lut[that code]), so that D + S reproduces it.

Naive-LoRA (naive_lora below): the rank-r factors whose product is the
truncated SVD of the residual E = W - W_hat, the approximation of least
Frobenius error (Eckart-Young).

Sources, by page (title, then section):
  * "SLiM: One-shot Quantization and Sparsity with Low-rank Approximation for
    LLM Weight Compression" -- review highlights, SLiM-LoRA bullet: Naive-LoRA
    minimises the plain error norm between the original and the compressed
    weight matrix (the saliency-weighted SLiM-LoRA needs calibration data and
    is not here).
  * "SqueezeLLM: Dense-and-Sparse Quantization" -- Approach: non-uniform LUT
    quantization whose centroids come from k-means over each output channel's
    weights, with outliers (and sensitive weights) kept apart in a
    full-precision CSR matrix, 0.45 % in total.  Measured-effects table: the
    sensitivity-agnostic clustering (plain k-means) is one of the ablations.
    The Fisher weighting itself needs gradients and data and is not here.

Readings where the page is silent (each one also listed with the design
notes): outliers by magnitude over the whole layer; the evenly spaced
initialisation, the tie rules and the stopping rule above; an outlier's dense
code.  Arithmetic: weights are fp16, so every sum of them is an exact integer
multiple of 2^-24; the sums are kept as such integers (exact in any order, for
|w| < 8192 and K <= 28672), a centroid is that sum over the count in fp64 (one
rounding), boundaries are (c_j + c_(j+1)) / 2 in fp64, and every comparison is
exact.  The fp64 -> fp16 rounding follows the format's definition.
"""
from __future__ import annotations

import numpy as np

FIX = float(1 << 24)  # fp16 values are integer multiples of 2^-24


def round_to_f16(v) -> np.ndarray:
    """Nearest fp16 value (ties to even) of fp64 values inside the fp16 range,
    from the definition: spacing 2^(e - 10), e the exponent (>= -14)."""
    v = np.asarray(v, dtype=np.float64)
    _, e = np.frexp(v)
    e = np.maximum(e - 1, -14)
    sp = np.ldexp(1.0, e - 10)
    return np.rint(v / sp) * sp


def select_outliers(W, n_out: int) -> np.ndarray:
    """Boolean mask [N, K] of the n_out largest |w|, ties to the lower row-major index."""
    a = np.abs(np.asarray(W, dtype=np.float16).astype(np.float64)).ravel()
    order = np.lexsort((np.arange(a.size), -a))  # by -|w|, then by index
    mask = np.zeros(a.size, dtype=bool)
    mask[order[:n_out]] = True
    return mask.reshape(np.asarray(W).shape)


def kmeans_row(v16, k: int, max_iter: int):
    """Lloyd's iterations on one row's dense weights (fp16 array); returns the fp64 centroids."""
    v = np.asarray(v16, dtype=np.float16).astype(np.float64)
    if v.size == 0:
        return np.zeros(k)
    q = np.rint(v * FIX).astype(np.int64)          # exact integers
    mn, mx = v.min() + 0.0, v.max() + 0.0             # a -0 bound counts as +0
    c = mn + ((mx - mn) * (2 * np.arange(k) + 1)) / (2 * k)
    for _ in range(max_iter):
        b = (c[:-1] + c[1:]) * 0.5                 # boundaries
        idx = np.searchsorted(b, v, side="left")   # number of boundaries < v
        sums = np.zeros(k, dtype=np.int64)
        np.add.at(sums, idx, q)
        cnt = np.bincount(idx, minlength=k)
        new = c.copy()
        nz = cnt > 0
        new[nz] = (sums[nz].astype(np.float64) / cnt[nz]) / FIX
        if np.array_equal(new, c):
            break
        c = new
    return c


def nearest_code(v, lut16) -> np.ndarray:
    """Code of the nearest LUT value (lower code on a tie); lut16 sorted ascending."""
    l = np.asarray(lut16, dtype=np.float16).astype(np.float64)
    b = (l[:-1] + l[1:]) * 0.5
    return np.searchsorted(b, np.asarray(v, dtype=np.float64), side="left").astype(np.uint8)


def fit_lut(W, bits: int, n_out: int, max_iter: int):
    """codes uint8 [N, K], lut fp16 [N, 2^b], CSR (row_ptr int32 [N+1], col int32, val fp16)."""
    W16 = np.asarray(W, dtype=np.float16)
    N, K = W16.shape
    k = 1 << bits
    out = select_outliers(W16, n_out)
    codes = np.zeros((N, K), dtype=np.uint8)
    lut = np.zeros((N, k), dtype=np.float16)
    rows, cols, vals = [], [], []
    for n in range(N):
        dense = ~out[n]
        c = kmeans_row(W16[n, dense], k, max_iter)
        l16 = round_to_f16(c).astype(np.float16)
        lut[n] = l16
        w = W16[n].astype(np.float64)
        codes[n] = nearest_code(np.where(dense, w, 0.0), l16)
        oc = np.flatnonzero(out[n])
        for j in oc:
            rows.append(n)
            cols.append(j)
            vals.append(round_to_f16(w[j] - float(l16[codes[n, j]])))
    row_ptr = np.zeros(N + 1, dtype=np.int32)
    np.cumsum(np.bincount(np.asarray(rows, dtype=np.int64), minlength=N), out=row_ptr[1:])
    return (codes, lut, row_ptr, np.asarray(cols, dtype=np.int32),
            np.asarray(vals, dtype=np.float64).astype(np.float16))


# ---------------------------------------------------------------------------
# Integer formats: magnitude masks and the SLiM-Quant clip search
# ---------------------------------------------------------------------------
#
# "SLiM: One-shot Quantization and Sparsity with Low-rank Approximation for LLM
# Weight Compression" -- review highlights: symmetric weight quantization that
# clips the weights before rounding to the nearest integer, the clipping
# threshold found by a grid search (the page's probabilistic formulation has
# lost its equations).  Rebuttal "Unstructured vs. 2:4 Sparsity": 2:4 and
# unstructured masks.  "Compressing Large Language Models by Joint
# Sparsification and Quantization", Approach: unstructured sparsity with
# quantization.  Pruning metrics that need activations (Wanda, SAR) are out;
# the data-free mask keeps the largest magnitudes.
#
# Readings: per output channel (row) a scale s = fp16(i * max|w| / (qmax * G))
# for the grid point i in 1..G (the clipping threshold i/G of the row's largest
# kept magnitude; the division in fp64, then rounded to fp16), codes
# q = clamp(rint(w / s), -qmax, qmax) with qmax = 2^(b-1) - 1, and the grid point
# with the smallest squared error sum (w - s q)^2 over the kept weights wins
# (the lower i on a tie); the errors are exact integers in units of 2^-48.
# Masks: 2:4 keeps the two largest |w| of each group of four consecutive
# weights, "half" keeps the floor(K/2) largest of each row; ties to the lower
# index.  Dropped weights get q = 0.

def magnitude_mask(W, kind: str) -> np.ndarray:
    """keep uint8 [N, K] of the data-free mask ('2:4' or 'half')."""
    a = np.abs(np.asarray(W, dtype=np.float16).astype(np.float64))
    N, K = a.shape
    keep = np.zeros((N, K), dtype=np.uint8)
    if kind == "2:4":
        for n in range(N):
            for g in range(K // 4):
                grp = a[n, 4 * g:4 * g + 4]
                order = sorted(range(4), key=lambda t: (-grp[t], t))
                keep[n, 4 * g + order[0]] = keep[n, 4 * g + order[1]] = 1
    elif kind == "half":
        for n in range(N):
            order = np.lexsort((np.arange(K), -a[n]))
            keep[n, order[:K // 2]] = 1
    else:
        keep[:] = 1
    return keep


def clip_search_row(w16, kept, bits: int, grid: int):
    """(scale fp16, q int8 [K]) of one row by the grid search above."""
    qmax = (1 << (bits - 1)) - 1
    w = np.asarray(w16, dtype=np.float16).astype(np.float64)
    k = np.asarray(kept, dtype=bool)
    q = np.zeros(w.size, dtype=np.int64)
    m = float(np.abs(w[k]).max()) if k.any() else 0.0
    wi = [int(v) for v in np.rint(w[k] * FIX).astype(np.int64)]
    best = None
    for i in range(1, grid + 1):
        s = float(round_to_f16((i * m) / (qmax * grid)))
        if s == 0.0:
            continue
        qi = np.clip(np.rint(w[k] / s), -qmax, qmax).astype(np.int64)
        si = int(round(s * FIX))
        err = sum((a - si * int(b)) ** 2 for a, b in zip(wi, qi))
        if best is None or err < best[0]:
            best = (err, s, qi)
    if best is None:
        return np.float16(0.0), q.astype(np.int8)
    q[k] = best[2]
    return np.float16(best[1]), q.astype(np.int8)


def fit_int(W, bits: int, mask: str, grid: int):
    """qvals int8 [N, K], row_scale fp16 [N], keep uint8 [N, K] (all ones without a mask)."""
    W16 = np.asarray(W, dtype=np.float16)
    keep = magnitude_mask(W16, mask)
    N, K = W16.shape
    q = np.zeros((N, K), dtype=np.int8)
    s = np.zeros(N, dtype=np.float16)
    for n in range(N):
        s[n], q[n] = clip_search_row(W16[n], keep[n], bits, grid)
    return q, s, keep


# ---------------------------------------------------------------------------
# AbsMax group quantization of the low-rank factors
# ---------------------------------------------------------------------------
#
# "SLiM" page, review highlights: the low-rank adapters are quantized with an
# AbsMax group scheme, group size 128.  Readings: 4-bit codes, groups of `group`
# consecutive entries along the first axis of the factor as stored logically
# (L [K, r]: along K for each rank column; R [r, N]: along r for each output
# column), scale = fp16(max|v| / 7) (fp64 division, nearest-even fp16),
# q = clamp(rint(v / scale), -8, 7) in fp64; an all-zero group gets scale 0, q 0.

def absmax_groups(F16, group: int, dtype: str = "f16"):
    """q int8 [R, C], scale fp16 [ceil(R / group), C] of a factor given as fp16
    values or bf16 bit patterns."""
    if dtype == "bf16":
        u = np.asarray(F16, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        v = u.view(np.float32).astype(np.float64)
    else:
        v = np.asarray(F16, dtype=np.float16).astype(np.float64)
    R, C = v.shape
    ng = -(-R // group)
    q = np.zeros((R, C), dtype=np.int8)
    sc = np.zeros((ng, C), dtype=np.float16)
    for g in range(ng):
        blk = v[g * group:(g + 1) * group]
        s = round_to_f16(np.abs(blk).max(axis=0) / 7.0)
        sc[g] = s.astype(np.float16)
        for c in range(C):
            if s[c] > 0:
                q[g * group:(g + 1) * group, c] = np.clip(np.rint(blk[:, c] / s[c]), -8, 7).astype(np.int8)
    return q, sc


def naive_lora(E, rank: int):
    """Naive-LoRA factors of the residual E [N, K] = W - W_hat (rows = output
    channels), SLiM page, review highlights, SLiM-LoRA bullet: with the SVD
    E = U diag(s) V^T (s descending), (L R)^T = U_r diag(s_r) V_r^T, the
    rank-r approximation of least Frobenius (and spectral) error.  The split
    of diag(s_r) between the factors is not given by the page; this reading
    gives each factor its square root:
        L = V_r diag(sqrt(s_r))   [K, rank]      R = diag(sqrt(s_r)) U_r^T   [rank, N]
    so that L^T L = R R^T = diag(s_r).  Ranks past min(N, K) get zero columns.
    Returns L, R (float64) and s_r."""
    E = np.asarray(E, dtype=np.float64)
    N, K = E.shape
    U, s, Vt = np.linalg.svd(E, full_matrices=False)
    r = min(rank, s.size)
    sq = np.sqrt(s[:r])
    L = np.zeros((K, rank))
    R = np.zeros((rank, N))
    L[:, :r] = Vt[:r].T * sq
    R[:r] = (U[:, :r] * sq).T
    sv = np.zeros(rank)
    sv[:r] = s[:r]
    return L, R, sv
