"""The five workloads at full size on the GPU, checked on sampled rows.

The oracle reconstructs only the sampled rows (first and last tile, plus a
seeded random sample), at the decode batches each workload names and in the
launch configuration the benchmark uses.
"""
import sys

import numpy as np
import pytest

import oracle
from gpu_util import check_bound, gpu_layer, to_device_x, torch_cuda
from synth.layers import CONFIGS, make_layer, make_x

pytestmark = pytest.mark.gpu

CASES = [(cfg, li) for cfg in range(1, 6) for li in range(len(CONFIGS[cfg]["layers"]))]


def sample_rows(N, seed):
    r = np.random.default_rng(seed)
    rows = set(range(0, min(N, 64))) | set(range(max(0, N - 64), N))
    rows |= set(r.choice(N, size=min(N, 128), replace=False).tolist())
    return np.array(sorted(rows))


@pytest.mark.parametrize("cfg,li", CASES, ids=[f"cfg{c}-{CONFIGS[c]['layers'][l][0]}" for c, l in CASES])
def test_full_size_sampled(cfg, li):
    torch = torch_cuda()
    Ms = [m for m in CONFIGS[cfg]["M"] if m <= 32]
    layer = make_layer(cfg, li, M_for_clamp=max(Ms))
    rows = sample_rows(layer.N, 100 * cfg + li)
    mod = gpu_layer(layer, max_M=max(CONFIGS[cfg]["M"]))
    # debug planes on the sampled rows, bit-exact
    print("full", layer.name, "debug", file=sys.stderr, flush=True)
    D16, S16, L32, R32 = mod.debug_dequant()
    torch.cuda.synchronize()
    ridx = torch.from_numpy(rows).cuda()
    d, s, _, _ = oracle.debug_planes(layer, rows)
    assert np.array_equal(D16[ridx].cpu().numpy().view(np.uint16), d.view(np.uint16))
    assert np.array_equal(S16[ridx].cpu().numpy().view(np.uint16), s.view(np.uint16))
    del D16, S16, L32, R32
    for M in CONFIGS[cfg]["M"]:
        x = make_x(cfg, li, M)
        print("full", layer.name, "M", M, file=sys.stderr, flush=True)
        y = mod.forward(to_device_x(x, layer.x_dtype))
        torch.cuda.synchronize()
        check_bound(y.cpu().numpy().astype(np.float64), layer, x, rows=rows, what=f"{layer.name} M={M}")
    mod.close()
