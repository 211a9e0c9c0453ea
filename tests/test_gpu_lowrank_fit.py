"""Naive-LoRA factors on the GPU (cl_fit_lowrank) against the oracle's exact
truncated SVD, through the C ABI (needs an MI355X).

The fitter iterates on a random subspace in fp32, so it matches the exact
truncation where the spectrum has a gap after the rank (products of the
factors and singular values within 1e-4 relative), and comes within 1 % of
the least possible error (Eckart-Young) on a flat, noise-like residual.  End
to end: W -> LUT fit -> residual -> factors -> pack -> forward, checked
against the oracle's forward of the packed layer, with a smaller total error
than the dense + sparse part alone.
"""
import sys

import numpy as np
import pytest

import compressed_linear_amd as cla
from oracle import fit_oracle as F
from gpu_util import check_bound, gpu_forward, torch_cuda
from synth.layers import LogicalLayer

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def _fit(E, rank, oversample=16, iters=8, seed=3):
    torch = torch_cuda()
    Ed = torch.from_numpy(np.ascontiguousarray(E, dtype=np.float32)).cuda()
    L, R, s = cla.fit_lowrank(Ed, rank, oversample, iters, seed)
    torch.cuda.synchronize()
    return L.cpu().numpy().astype(np.float64), R.cpu().numpy().astype(np.float64), s.astype(np.float64)


def _orth(r, n, k):
    q, _ = np.linalg.qr(r.normal(0, 1, (n, k)))
    return q


@pytest.mark.parametrize("N,K,rank", [(700, 500, 20), (300, 1100, 64), (129, 65, 8)])
def test_gapped_spectrum_matches_truncated_svd(N, K, rank):
    r = np.random.default_rng(N + K)
    n = min(N, K)
    s = np.concatenate([np.linspace(10.0, 1.0, rank), 0.05 * np.exp(-np.arange(n - rank) / 30.0)])
    E = (_orth(r, N, n) * s) @ _orth(r, K, n).T
    say("gapped", N, K, rank)
    L, R, sv = _fit(E, rank)
    Lo, Ro, so = F.naive_lora(E, rank)
    P, Po = (L @ R).T, (Lo @ Ro).T
    assert np.linalg.norm(P - Po) <= 1e-4 * np.linalg.norm(Po), np.linalg.norm(P - Po) / np.linalg.norm(Po)
    assert np.allclose(sv, so, rtol=1e-4, atol=0)
    # the square-root split: L^T L = R R^T = diag(s), up to the fp32 products
    assert np.allclose(L.T @ L, np.diag(so), atol=1e-3 * so[0]) and np.allclose(R @ R.T, np.diag(so), atol=1e-3 * so[0])


def test_flat_residual_near_optimal():
    # quantization-noise-like residual: no gap, so the subspace is not unique;
    # the error must still be within 1 % of the least possible
    r = np.random.default_rng(11)
    N, K, rank = 1024, 768, 64
    E = r.normal(0, 1, (N, K)) * (1 + 0.3 * r.random((1, K)))
    say("flat", N, K, rank)
    L, R, sv = _fit(E, rank, oversample=32, iters=10)
    Lo, Ro, so = F.naive_lora(E, rank)
    err, best = np.linalg.norm(E - (L @ R).T), np.linalg.norm(E - (Lo @ Ro).T)
    assert err <= 1.01 * best, (err, best)
    assert np.all(sv <= so * (1 + 1e-4))  # estimates from a subspace never exceed the true values


def test_rank_past_min_dimension_and_low_rank_input():
    r = np.random.default_rng(5)
    E = r.normal(0, 1, (40, 3)) @ r.normal(0, 1, (3, 30))  # rank 3
    say("rank 5 of a rank-3 matrix")
    L, R, sv = _fit(E, 5, oversample=4, iters=3)
    assert np.linalg.norm((L @ R).T - E) <= 1e-4 * np.linalg.norm(E)
    assert np.all(sv[3:] <= 1e-4 * sv[0])
    L, R, sv = _fit(E, 40, oversample=0, iters=1)  # rank past min(N, K) = 30
    assert np.linalg.norm((L @ R).T - E) <= 1e-4 * np.linalg.norm(E) and np.all(L[:, 30:] == 0) and np.all(R[30:] == 0)


def _dequant_lut(codes, lut, rp, col, val):
    D = np.take_along_axis(lut.astype(np.float64), codes.astype(np.int64), axis=1)
    S = np.zeros_like(D)
    for n in range(D.shape[0]):
        for e in range(rp[n], rp[n + 1]):
            S[n, col[e]] += float(val[e])
    return D + S


@pytest.mark.parametrize("lr", ["fp16", "bf16"])
def test_fit_pack_forward(lr):
    torch = torch_cuda()
    r = np.random.default_rng(21)
    N, K, rank = 512, 1088, 32
    W = (r.normal(0, 0.02, (N, K)) + 0.01 * r.normal(0, 1, (N, 4)) @ r.normal(0, 1, (4, K))).astype(np.float16)
    Wd = torch.from_numpy(W.view(np.int16)).view(torch.float16).cuda()
    codes, lut, rp, col, val = (t.cpu().numpy() for t in cla.fit_lut(Wd, 3, N * K // 200, 30))
    W_hat = _dequant_lut(codes, lut, rp, col, val)
    E = W.astype(np.float64) - W_hat
    say("fit -> pack -> forward", lr)
    L, R, sv = _fit(E, rank)
    if lr == "fp16":
        Lq, Rq = L.astype(np.float16), R.astype(np.float16)
    else:
        from synth.layers import bf16_bits_from_f32
        Lq, Rq = bf16_bits_from_f32(L), bf16_bits_from_f32(R)
    lay = LogicalLayer(K=K, N=N, dense="lut3", codes=codes, lut=lut, csr_row_ptr=rp, csr_col=col, csr_val=val,
                       lr=lr, rank=rank, L=Lq, R=Rq)
    # the factors lower the error of the compressed matrix (by at least the
    # part the exact truncation removes, less its fp32/16-bit rounding)
    Lo, Ro, so = F.naive_lora(E, rank)
    Lf = Lq.astype(np.float64) if lr == "fp16" else (Lq.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    Rf = Rq.astype(np.float64) if lr == "fp16" else (Rq.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    e0, e1, eo = np.linalg.norm(E), np.linalg.norm(E - (Lf @ Rf).T), np.linalg.norm(E - (Lo @ Ro).T)
    assert e1 < e0 and e1 <= eo + 0.02 * (e0 - eo), (e0, e1, eo)
    for M in (1, 4, 40):
        x = r.normal(0, 1, (M, K)).astype(np.float16)
        check_bound(gpu_forward(lay, x), lay, x, what=f"fitted {lr} M={M}")
