"""Seeded synthetic layers and activations.

Every array here is a *logical* (unpacked) input of the forward: codes and
LUTs, integer values and per-row scales, keep masks, CSR outliers,
low-rank factors, the activation clamp and the activations.  Random draws
use ``numpy.random.Generator(PCG64(SeedSequence([2026, cfg, layer, stream])))``
with one stream per quantity, so each array is reproducible on its own:

    0 codes / integer values      4 CSR values
    1 LUT centroids / scales      5 low-rank L
    2 mask                        6 low-rank R
    3 CSR positions               7 activations (key also holds M)
                                  8 per-channel activation factors

Rounding to fp16 uses numpy's round-to-nearest-even cast; bf16 values are
drawn in fp64, cast to fp32 and rounded to bf16 (nearest, ties to even).
numpy has no bf16 dtype, so bf16 arrays are carried as uint16 bit patterns.

The two quantisers used to *produce* integer inputs (AbsMax int4 for the
low-rank factors, per-row symmetric int8 for the dense part) are input
synthesis: the forward never quantises, it only consumes (q, scale).
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Optional

import numpy as np

ROOT_SEED = 2026

# Stream ids of the seed sequence.
S_CODES, S_LUT, S_MASK, S_CSR_POS, S_CSR_VAL, S_L, S_R, S_X, S_XSCALE = range(9)

# The six ways to keep 2 of 4 consecutive weights.
PAIRS_2_4 = np.array([(0, 1), (0, 2), (0, 3), (1, 2), (1, 3), (2, 3)], dtype=np.int64)


def _rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([ROOT_SEED, *key])))


def bf16_bits_from_f32(a) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); return the uint16 bits."""
    f = np.ascontiguousarray(np.asarray(a, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    nan = np.isnan(f)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    if nan.any():
        r = np.where(nan, np.uint16(0x7FC0), r)
    return r


def f32_from_bf16_bits(b) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to fp32 values; exact."""
    u = np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32)


@dataclass
class LogicalLayer:
    """One compressed linear layer in logical (unpacked) form.

    W_hat is [N, K]: N = out_features (rows), K = in_features.
      dense   'lut3' | 'lut4'  codes uint8 [N, K] in 0..2^b-1, lut fp16 [N, 2^b]
              'int4' | 'int8'  qvals int8 [N, K], row_scale fp16 [N]
      mask    'none' | '2:4' | 'bitmap'; keep uint8 [N, K] (1 = kept)
      CSR     row_ptr int32 [N+1], col int32 [nnz], val fp16 [nnz]
      lr      'none' | 'fp16' | 'bf16' | 'int4'
              fp16: L fp16 [K, r], R fp16 [r, N]
              bf16: L, R uint16 bf16 bits
              int4: L, R int8 codes in -8..7; L_scale fp16 [ceil(K/g), r],
                    R_scale fp16 [ceil(r/g), N]
      act_clamp  fp16 scalar (np.float16) or None
      xscale_ch  int32 [n] strictly increasing input channels whose activations
                 are scaled (SLiM's output-error variant), or None
      xscale     fp16 [n] the factor each of those activations is multiplied by
                 (1/alpha, in (0, 1]), or None
      x_dtype    'f16' | 'bf16'
    """

    K: int
    N: int
    dense: str
    mask: str = "none"
    codes: Optional[np.ndarray] = None
    lut: Optional[np.ndarray] = None
    qvals: Optional[np.ndarray] = None
    row_scale: Optional[np.ndarray] = None
    keep: Optional[np.ndarray] = None
    csr_row_ptr: Optional[np.ndarray] = None
    csr_col: Optional[np.ndarray] = None
    csr_val: Optional[np.ndarray] = None
    lr: str = "none"
    rank: int = 0
    group: int = 128
    L: Optional[np.ndarray] = None
    R: Optional[np.ndarray] = None
    L_scale: Optional[np.ndarray] = None
    R_scale: Optional[np.ndarray] = None
    act_clamp: Optional[np.float16] = None
    xscale_ch: Optional[np.ndarray] = None
    xscale: Optional[np.ndarray] = None
    x_dtype: str = "f16"
    name: str = ""
    meta: dict = field(default_factory=dict)

    @property
    def bits(self) -> int:
        return {"lut3": 3, "lut4": 4, "int4": 4, "int8": 8}[self.dense]

    @property
    def nnz(self) -> int:
        return 0 if self.csr_col is None else int(self.csr_col.shape[0])

    def with_(self, **kw) -> "LogicalLayer":
        return replace(self, **kw)


# ---------------------------------------------------------------------------
# Building blocks (all draws, no forward arithmetic)
# ---------------------------------------------------------------------------

def draw_lut_codes(rng_codes, rng_lut, N, K, bits, sigma=0.02, sort=True):
    codes = rng_codes.integers(0, 1 << bits, size=(N, K), dtype=np.uint8)
    cent = rng_lut.normal(0.0, sigma, size=(N, 1 << bits))
    if sort:
        cent = np.sort(cent, axis=1)
    return codes, cent.astype(np.float16)


def draw_csr(rng_pos, rng_val, N, K, density=0.0045, sigma=0.2, nnz=None):
    """Outliers at uniform random distinct positions, sorted row-major."""
    total = N * K
    if nnz is None:
        nnz = int(round(density * total))
    nnz = min(nnz, total)
    if nnz == 0:
        pos = np.zeros(0, dtype=np.int64)
    else:
        pos = np.sort(rng_pos.choice(total, size=nnz, replace=False).astype(np.int64))
    rows = pos // K
    cols = (pos % K).astype(np.int32)
    counts = np.bincount(rows, minlength=N)
    row_ptr = np.zeros(N + 1, dtype=np.int64)
    np.cumsum(counts, out=row_ptr[1:])
    vals = rng_val.normal(0.0, sigma, size=nnz).astype(np.float16)
    return row_ptr.astype(np.int32), cols, vals


def draw_csr_skewed(rng_pos, rng_val, N, K, density=0.0045, hot_frac=0.01, hot_share=0.5, sigma=0.2):
    """Stress pattern: `hot_share` of the outliers sit in `hot_frac` of the rows."""
    nnz = int(round(density * N * K))
    n_hot_rows = max(1, int(round(hot_frac * N)))
    hot_rows = np.sort(rng_pos.choice(N, size=n_hot_rows, replace=False))
    n_hot = min(int(round(hot_share * nnz)), n_hot_rows * K)
    hot_cells = rng_pos.choice(n_hot_rows * K, size=n_hot, replace=False)
    hot_pos = hot_rows[hot_cells // K].astype(np.int64) * K + (hot_cells % K)
    mask = np.zeros(N * K, dtype=bool)
    mask[hot_pos] = True
    rest = nnz - n_hot
    free = np.flatnonzero(~mask)
    cold_pos = rng_pos.choice(free, size=min(rest, free.size), replace=False)
    pos = np.sort(np.concatenate([hot_pos, cold_pos]))
    rows = pos // K
    cols = (pos % K).astype(np.int32)
    row_ptr = np.zeros(N + 1, dtype=np.int64)
    np.cumsum(np.bincount(rows, minlength=N), out=row_ptr[1:])
    vals = rng_val.normal(0.0, sigma, size=pos.size).astype(np.float16)
    return row_ptr.astype(np.int32), cols, vals


def draw_act_scale(rng, K, frac=0.01, alpha_max=4.0):
    """About `frac` of the K input channels, uniform at random, each with a
    factor alpha drawn uniformly from [1, alpha_max]; returns the sorted
    channels (int32) and the activation factors fp16(1/alpha)."""
    n = int(round(frac * K))
    ch = np.sort(rng.choice(K, size=n, replace=False)).astype(np.int32)
    alpha = rng.uniform(1.0, alpha_max, size=n)
    return ch, (1.0 / alpha).astype(np.float16)


def draw_mask_2_4(rng_mask, N, K):
    assert K % 4 == 0
    choice = rng_mask.integers(0, 6, size=(N, K // 4))
    pairs = PAIRS_2_4[choice]  # [N, K/4, 2]
    keep = np.zeros((N, K // 4, 4), dtype=np.uint8)
    np.put_along_axis(keep, pairs, 1, axis=2)
    return keep.reshape(N, K)


def draw_mask_half(rng_mask, N, K):
    """Exactly floor(K/2) kept per row, a uniform random subset of each row."""
    base = np.zeros((N, K), dtype=np.uint8)
    base[:, : K // 2] = 1
    return rng_mask.permuted(base, axis=1)


def absmax_int4_groups(v: np.ndarray, group: int):
    """AbsMax int4 codes of `v` in groups of `group` along axis 0.

    scale = fp16(max|v| / 7) per (group, column); q = clamp(rint(v / scale), -8, 7)
    using the fp16-rounded scale; an all-zero group gets scale 0 and q = 0.
    Used only to synthesise int4 factors.
    """
    rows, cols = v.shape
    ng = -(-rows // group)
    scale = np.zeros((ng, cols), dtype=np.float16)
    q = np.zeros((rows, cols), dtype=np.int8)
    for g in range(ng):
        blk = v[g * group:(g + 1) * group]
        s = (np.abs(blk).max(axis=0) / 7.0).astype(np.float16)
        scale[g] = s
        sf = s.astype(np.float64)
        with np.errstate(divide="ignore", invalid="ignore"):
            qq = np.where(sf > 0, np.rint(blk / np.where(sf > 0, sf, 1.0)), 0.0)
        q[g * group:(g + 1) * group] = np.clip(qq, -8, 7).astype(np.int8)
    return q, scale


def rowwise_int8(w: np.ndarray, keep: np.ndarray):
    """Per-row symmetric int8 codes of the kept weights (input synthesis only)."""
    kept_abs = np.where(keep.astype(bool), np.abs(w), 0.0)
    s = (kept_abs.max(axis=1) / 127.0).astype(np.float16)
    sf = s.astype(np.float64)[:, None]
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where(sf > 0, np.rint(w / np.where(sf > 0, sf, 1.0)), 0.0)
    q = np.clip(q, -127, 127)
    q = np.where(keep.astype(bool), q, 0).astype(np.int8)
    return q, s


# ---------------------------------------------------------------------------
# The five workloads
# ---------------------------------------------------------------------------

# (name, K, N) per layer; M values decode (<= 32) and prefill.
CONFIGS = {
    1: dict(desc="4096x4096 LUT3 + CSR, batch 1",
            layers=[("4096x4096", 4096, 4096)], M=[1]),
    2: dict(desc="LLaMA-7B decode layer set, LUT4 + CSR, batch 1",
            layers=[("qkv", 4096, 12288), ("o", 4096, 4096), ("gate", 4096, 11008),
                    ("up", 4096, 11008), ("down", 11008, 4096)], M=[1]),
    3: dict(desc="SLiM-style INT4 2:4 + int4 low-rank r128",
            layers=[("up", 4096, 11008), ("down", 11008, 4096)], M=[1, 8, 16]),
    4: dict(desc="JSQ-style INT8 50% bitmap + activation clamp",
            layers=[("up", 6656, 17920), ("down", 17920, 6656)], M=[16]),
    5: dict(desc="LLaMA-70B LUT3 + CSR + bf16 low-rank r64",
            layers=[("qkv", 8192, 10240), ("up", 8192, 28672), ("down", 28672, 8192)],
            M=[1, 4, 16, 32, 2048]),
}


def config_layers(cfg: int):
    return CONFIGS[cfg]["layers"]


def _layer_index(cfg: int, layer) -> int:
    if isinstance(layer, int):
        return layer
    names = [n for n, _, _ in CONFIGS[cfg]["layers"]]
    return names.index(layer)


def make_x(cfg: int, layer, M: int, K: Optional[int] = None) -> np.ndarray:
    """Activations [M, K]: fp16 (np.float16) or bf16 bits (np.uint16)."""
    li = _layer_index(cfg, layer)
    if K is None:
        K = CONFIGS[cfg]["layers"][li][1]
    rng = _rng(cfg, li, S_X, M)
    base = rng.normal(0.0, 1.0, size=(M, K))
    if cfg == 3:
        nch = int(round(0.001 * K))
        ch = rng.choice(K, size=nch, replace=False)
        base[:, ch] *= 20.0
        return base.astype(np.float16)
    if cfg == 4:
        out = rng.random(size=(M, K)) < 0.005
        big = rng.normal(0.0, 30.0, size=(M, K))
        base = np.where(out, big, base)
        return base.astype(np.float16)
    if cfg == 5:
        return bf16_bits_from_f32(base.astype(np.float32))
    return base.astype(np.float16)


def clamp_value_for(x16: np.ndarray) -> np.float16:
    """Per-layer clamp: fp16 of the 99.9th percentile of |x| over the batch."""
    v = np.abs(x16.astype(np.float64)).ravel()
    return np.float16(np.quantile(v, 0.999))


def make_layer(cfg: int, layer, K: Optional[int] = None, N: Optional[int] = None,
               M_for_clamp: int = 16) -> LogicalLayer:
    """The seeded logical layer `layer` of workload `cfg`.

    K and N override the shape (same distributions), for parity tests at
    sizes the oracle finishes in seconds.
    """
    li = _layer_index(cfg, layer)
    name, K0, N0 = CONFIGS[cfg]["layers"][li]
    K = K0 if K is None else K
    N = N0 if N is None else N
    r = lambda s: _rng(cfg, li, s)
    tag = f"cfg{cfg}/{name}/{K}x{N}"

    if cfg in (1, 2, 5):
        bits = 3 if cfg in (1, 5) else 4
        codes, lut = draw_lut_codes(r(S_CODES), r(S_LUT), N, K, bits)
        rp, col, val = draw_csr(r(S_CSR_POS), r(S_CSR_VAL), N, K)
        lay = LogicalLayer(K=K, N=N, dense=f"lut{bits}", codes=codes, lut=lut,
                           csr_row_ptr=rp, csr_col=col, csr_val=val,
                           x_dtype="bf16" if cfg == 5 else "f16", name=tag)
        if cfg == 5:
            rank = 64
            Lf = r(S_L).normal(0.0, 0.01, size=(K, rank)).astype(np.float32)
            Rf = r(S_R).normal(0.0, 0.01, size=(rank, N)).astype(np.float32)
            lay = lay.with_(lr="bf16", rank=rank, L=bf16_bits_from_f32(Lf), R=bf16_bits_from_f32(Rf))
        return lay

    if cfg == 3:
        keep = draw_mask_2_4(r(S_MASK), N, K)
        q = r(S_CODES).integers(-8, 8, size=(N, K), dtype=np.int8)
        q = np.where(keep.astype(bool), q, 0).astype(np.int8)
        scale = np.full(N, np.float16(0.02 / 7.0), dtype=np.float16)
        rank, group = 128, 128
        Lf = r(S_L).normal(0.0, 0.01, size=(K, rank))
        Rf = r(S_R).normal(0.0, 0.01, size=(rank, N))
        Lq, Ls = absmax_int4_groups(Lf, group)
        Rq, Rs = absmax_int4_groups(Rf, group)
        return LogicalLayer(K=K, N=N, dense="int4", mask="2:4", qvals=q, row_scale=scale, keep=keep,
                            lr="int4", rank=rank, group=group, L=Lq, R=Rq, L_scale=Ls, R_scale=Rs,
                            x_dtype="f16", name=tag)

    if cfg == 4:
        keep = draw_mask_half(r(S_MASK), N, K)
        w = r(S_CODES).normal(0.0, 0.02, size=(N, K))
        q, s = rowwise_int8(w, keep)
        x = make_x(cfg, li, M_for_clamp, K=K)
        c = clamp_value_for(x)
        return LogicalLayer(K=K, N=N, dense="int8", mask="bitmap", qvals=q, row_scale=s, keep=keep,
                            act_clamp=c, x_dtype="f16", name=tag, meta={"clamp_M": M_for_clamp})

    raise ValueError(f"unknown config {cfg}")


def with_act_scale(layer: LogicalLayer, seed: int = 0, frac: float = 0.01) -> LogicalLayer:
    """`layer` with about `frac` of its input channels scaled (seeded by `seed`
    and the layer's shape), the recipe of SLiM's output-error variant."""
    ch, f = draw_act_scale(_rng(layer.K, layer.N, S_XSCALE, seed), layer.K, frac)
    return layer.with_(xscale_ch=ch, xscale=f)


def empty_csr(N: int):
    return (np.zeros(N + 1, dtype=np.int32), np.zeros(0, dtype=np.int32), np.zeros(0, dtype=np.float16))
