"""CPU oracle of the compressed linear layer forward -- TEST INFRASTRUCTURE.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg
may import or run this module.  The HIP library never calls it and it
never calls the HIP library: the two share no code, no tables and no
helpers.  The only thing they share is the seeded input generator, which
holds none of the forward's arithmetic.

What it computes is a plain definition, written out in fp64:

    x'      = clamp(x, -c, c) if the layer carries a clamp c, else x
    x'[:,k] = rnd(x'[:,k] * f_k) on the scaled channels k, if any, where
              f_k = 1/alpha_k and rnd rounds to the activation type
    W_hat   = D + S + (L_hat R_hat)^T                       [N, K]
    y       = x' W_hat^T                                     [M, N]
    bound   = 1e-3 * |x'| |W_hat|^T                          (elementwise)

with
    D[n, k] = lut_n[code[n, k]]            (LUT formats)
            = q[n, k] * s_n                (integer formats)
            = 0 where the keep mask drops the weight
    S       = the fp16 outliers stored in CSR, at their (row, col)
    L_hat   = L (fp16/bf16) or q_L * scale (int4, AbsMax groups along K)
    R_hat   = R (fp16/bf16) or q_R * scale (int4, AbsMax groups along r)

Sources, by page (title, then section):
  * "SqueezeLLM: Dense-and-Sparse Quantization" -- Approach: non-uniform
    LUT (k-means centroid) codes for the dense part; outliers and sensitive
    weights kept apart in a full-precision CSR matrix.  Summary: 3/4-bit
    codes, outliers in an FP16 sparse format.
  * "SLiM: One-shot Quantization and Sparsity with Low-rank Approximation
    for LLM Weight Compression" -- review highlights: symmetric weight
    quantization with clipping and round-to-nearest (SLiM-Quant); low-rank
    adapters that compensate compression error (SLiM-LoRA); AbsMax group
    quantization of the adapters with group size 128.  Rebuttal section
    "Unstructured vs. 2:4 Sparsity": 2:4 semi-structured and unstructured
    masks.
  * "Compressing Large Language Models by Joint Sparsification and
    Quantization" -- Approach: unstructured sparsity combined with
    quantization; activation outliers clamped with one per-layer strength.
  * SLiM page, rebuttal section "Output Error Minimization in SLiM-Quant":
    the weights of about 1 % of the input channels (the most salient) are
    scaled up by a factor alpha and the matching activations are scaled
    down by the same factor while the layer runs.

Readings where the pages are silent (each one also listed with the design
notes): W_hat is [N, K] with rows = output channels, so "per row" LUTs and
scales belong to an output channel; D and S add (an outlier position keeps
its dense code as well); the clamp is symmetric, |x'| <= c; the int4 AbsMax
groups run along each factor's contraction axis; the output is fp32.  For
the channel scaling: the stored weights already carry alpha, the layer
stores the activation factor f = 1/alpha per scaled channel in fp16, the
clamp (when both are present) comes first, and a scaled activation is an
activation again, so x * f is rounded once, to nearest-even, to the
activation type (fp16 or bf16).

Parity status: every function below is pinned by CPU tests (hand-derived
closed forms, invariants, library-routine cross-checks, brute force); see
the test suite's oracle-pin module.
"""
from __future__ import annotations

import numpy as np

TOL_REL = 1e-3  # the forward's elementwise error bound, relative to |x'| |W_hat|^T


# ---------------------------------------------------------------------------
# element types
# ---------------------------------------------------------------------------

def _bf16_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> fp64, exactly (bf16 is the top half of fp32)."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def _act_to_f64(x, x_dtype: str) -> np.ndarray:
    if x_dtype == "bf16":
        return _bf16_to_f64(x)
    return np.asarray(x, dtype=np.float16).astype(np.float64)


# significand bits (with the leading one) and smallest normal exponent
_ACT_FORMATS = {"f16": (11, -14), "bf16": (8, -126)}


def round_to_act(v, x_dtype: str) -> np.ndarray:
    """Round fp64 values to the nearest value of the activation type, ties to
    even, from the definition of a binary floating-point format with p
    significand bits: the spacing of the values near v is 2^(e - p + 1), with
    e the exponent of v (not below the smallest normal one, which gives the
    subnormals).  Values are assumed inside the type's finite range."""
    p, emin = _ACT_FORMATS[x_dtype]
    v = np.asarray(v, dtype=np.float64)
    _, e = np.frexp(v)                  # v = m 2^e, 0.5 <= |m| < 1: exponent e - 1
    e = np.maximum(e - 1, emin)
    spacing = np.ldexp(1.0, e - (p - 1))
    return np.rint(v / spacing) * spacing  # exact: a power-of-two rescale, then rint (ties to even)


# ---------------------------------------------------------------------------
# step 1: activation clamp
# ---------------------------------------------------------------------------

def activations(layer, x) -> np.ndarray:
    """x' in fp64, [M, K].

    JSQ page, Approach: an activation editor clamps activation outliers with
    a per-layer strength.  Reading: one value c per layer, applied
    symmetrically, x' = min(max(x, -c), c); no clamp when the layer has none.
    Then the channel scaling of SLiM's output-error variant, if the layer
    has scaled channels (see the module docstring for its reading).
    """
    xf = _act_to_f64(x, layer.x_dtype)
    if xf.ndim == 1:
        xf = xf[None, :]
    c = getattr(layer, "act_clamp", None)
    if c is not None:
        cf = float(np.float16(c))
        xf = np.minimum(np.maximum(xf, -cf), cf)
    ch = getattr(layer, "xscale_ch", None)
    if ch is not None and len(ch):
        # SLiM page, "Output Error Minimization in SLiM-Quant": the activations
        # of the scaled channels are divided by alpha, i.e. multiplied by the
        # stored factor 1/alpha; the product is an activation of the layer's
        # input type again.
        f = np.asarray(layer.xscale, dtype=np.float16).astype(np.float64)
        cols = np.asarray(ch, dtype=np.int64)
        xf = xf.copy()
        xf[:, cols] = round_to_act(xf[:, cols] * f[None, :], layer.x_dtype)
    return xf


# ---------------------------------------------------------------------------
# step 2: dense part D
# ---------------------------------------------------------------------------

def _rows(layer, rows):
    return np.arange(layer.N) if rows is None else np.asarray(rows, dtype=np.int64)


def dense_plane(layer, rows=None) -> np.ndarray:
    """D[n, k] in fp64 for the selected rows.

    LUT formats (SqueezeLLM page, Approach): each weight is the centroid its
    code selects in the row's table, D[n, k] = lut[n, code[n, k]].
    Integer formats (SLiM page, highlights, SLiM-Quant): symmetric codes
    with a per-row scale, D[n, k] = q[n, k] * s[n] (the fp64 product is exact).
    Masks (SLiM rebuttal "Unstructured vs. 2:4 Sparsity"; JSQ Approach):
    a weight the mask drops is zero.
    """
    idx = _rows(layer, rows)
    if layer.dense in ("lut3", "lut4"):
        lut = np.asarray(layer.lut, dtype=np.float16).astype(np.float64)[idx]       # [n, 2^b]
        codes = np.asarray(layer.codes)[idx].astype(np.int64)                       # [n, K]
        D = np.take_along_axis(lut, codes, axis=1)
    elif layer.dense in ("int4", "int8"):
        q = np.asarray(layer.qvals)[idx].astype(np.float64)
        s = np.asarray(layer.row_scale, dtype=np.float16).astype(np.float64)[idx]
        D = q * s[:, None]
    else:
        raise ValueError(layer.dense)
    if layer.mask != "none":
        keep = np.asarray(layer.keep)[idx].astype(bool)
        D = np.where(keep, D, 0.0)
    return D


# ---------------------------------------------------------------------------
# step 3: sparse part S
# ---------------------------------------------------------------------------

def sparse_plane(layer, rows=None) -> np.ndarray:
    """S[n, k] in fp64: the CSR outliers at their positions, zero elsewhere.

    SqueezeLLM page, Approach: outliers and sensitive weights go into a
    full-precision sparse matrix in CSR form; the summary names fp16.
    Entries of one row are summed if a column repeats (the CSR definition).
    """
    idx = _rows(layer, rows)
    S = np.zeros((idx.size, layer.K), dtype=np.float64)
    if layer.csr_col is None or layer.nnz == 0:
        return S
    rp = np.asarray(layer.csr_row_ptr, dtype=np.int64)
    col = np.asarray(layer.csr_col, dtype=np.int64)
    val = np.asarray(layer.csr_val, dtype=np.float16).astype(np.float64)
    for i, n in enumerate(idx):
        a, b = rp[n], rp[n + 1]
        np.add.at(S[i], col[a:b], val[a:b])
    return S


# ---------------------------------------------------------------------------
# step 4: low-rank factors
# ---------------------------------------------------------------------------

def _dequant_groups(q, scale, group: int) -> np.ndarray:
    """q * scale with one scale per `group` consecutive entries along axis 0."""
    qf = np.asarray(q).astype(np.float64)
    sf = np.asarray(scale, dtype=np.float16).astype(np.float64)
    g_of_row = np.arange(qf.shape[0]) // group
    return qf * sf[g_of_row]


def lowrank_factors(layer):
    """(L_hat [K, r], R_hat [r, N]) in fp64, or (None, None) without a low-rank part.

    SLiM page, highlights: low-rank adapters compensate the compression
    error (SLiM-LoRA), and may be stored with AbsMax group quantization,
    group size 128 ("Low-rank adapter quantization").  Reading: groups run
    along each factor's contraction axis -- L along K for every rank column,
    R along r for every output column -- and a value is q * scale.
    """
    if layer.lr == "none" or layer.rank == 0:
        return None, None
    if layer.lr == "fp16":
        Lh = np.asarray(layer.L, dtype=np.float16).astype(np.float64)
        Rh = np.asarray(layer.R, dtype=np.float16).astype(np.float64)
    elif layer.lr == "bf16":
        Lh = _bf16_to_f64(layer.L)
        Rh = _bf16_to_f64(layer.R)
    elif layer.lr == "int4":
        Lh = _dequant_groups(layer.L, layer.L_scale, layer.group)
        Rh = _dequant_groups(layer.R, layer.R_scale, layer.group)
    else:
        raise ValueError(layer.lr)
    return Lh, Rh


# ---------------------------------------------------------------------------
# step 5: reconstruction and forward
# ---------------------------------------------------------------------------

def reconstruct(layer, rows=None) -> np.ndarray:
    """W_hat = D + S + (L_hat R_hat)^T, fp64, for the selected rows [n, K].

    SqueezeLLM page, Approach (dense-and-sparse: W = D + S) and SLiM page,
    highlights (a low-rank term added to the compressed weight).
    """
    idx = _rows(layer, rows)
    W = dense_plane(layer, idx) + sparse_plane(layer, idx)
    Lh, Rh = lowrank_factors(layer)
    if Lh is not None:
        W = W + (Lh @ Rh[:, idx]).T
    return W


def forward(layer, x, rows=None) -> np.ndarray:
    """y = x' W_hat^T in fp64, [M, n] for the selected output rows."""
    xp = activations(layer, x)
    W = reconstruct(layer, rows)
    return xp @ W.T


def bound(layer, x, rows=None) -> np.ndarray:
    """Elementwise tolerance 1e-3 * |x'| |W_hat|^T for the selected rows."""
    xp = activations(layer, x)
    W = reconstruct(layer, rows)
    return TOL_REL * (np.abs(xp) @ np.abs(W).T)


def forward_and_bound(layer, x, rows=None):
    """(y, bound) sharing one reconstruction."""
    xp = activations(layer, x)
    W = reconstruct(layer, rows)
    return xp @ W.T, TOL_REL * (np.abs(xp) @ np.abs(W).T)


# ---------------------------------------------------------------------------
# debug planes (bit-exact dequantisation check)
# ---------------------------------------------------------------------------

def debug_planes(layer, rows=None):
    """The unique fp16 / fp32 images of the parts of W_hat.

    D16 = fp16(D) with round-to-nearest-even (exact for LUT codes; for the
    integer formats q * s rounded once); S16 = the fp16 outliers at their
    positions; L32, R32 = fp32(L_hat), fp32(R_hat), which are exact.
    A sum D + S + LR in fp16 is not unique, so the parts stay separate.
    """
    idx = _rows(layer, rows)
    D16 = dense_plane(layer, idx).astype(np.float16)
    S16 = sparse_plane(layer, idx).astype(np.float16)
    Lh, Rh = lowrank_factors(layer)
    L32 = None if Lh is None else Lh.astype(np.float32)
    R32 = None if Rh is None else Rh.astype(np.float32)
    return D16, S16, L32, R32
