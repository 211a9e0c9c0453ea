"""Forwards recorded into a HIP graph and replayed (needs an MI355X).

Every replay, with new activations copied into the captured input between
replays and eager forwards of the same layer interleaved, must give bit for
bit the eager forward's output -- including layers whose decode launch
computes x' L_hat inside (their generation lives on the device) -- and stay
within the oracle's bound.
"""
import sys

import numpy as np
import pytest

import compressed_linear_amd as cla
from gpu_util import check_bound, to_device_x, torch_cuda
from synth.layers import make_layer, make_x, with_act_scale

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


CASES = [
    # (cfg, layer index, K, N, M, path)
    (5, 0, 1456, 190, 1, "auto"),        # bf16 LUT3 + rank 64: row kernel with the prologue inside
    (5, 0, 1456, 190, 8, "auto"),        # matrix-core decode with the prologue inside
    (3, 1, 768, 130, 1, "auto"),         # int4 2:4 + int4 rank 128, batch 1
    (3, 1, 768, 130, 16, "auto"),
    (2, 0, 1000, 150, 1, "auto"),        # no rank term
    (4, 0, 1280, 140, 16, "auto"),       # bitmap + clamp (split-K counters)
    (5, 0, 1456, 190, 40, "prefill"),    # prefill with the rank prologue
    (5, 0, 2600, 700, 1, "decode_stream"),  # batch-1 streaming kernel with the prologue inside
    (3, 1, 4160, 600, 1, "decode_stream"),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"cfg{c[0]}-M{c[4]}-{c[5]}")
def test_graph_replay_matches_eager(case):
    torch = torch_cuda()
    cfg, li, K, N, M, path = case
    layer = make_layer(cfg, li, K=K, N=N, M_for_clamp=max(M, 2))
    if cfg == 2:
        layer = with_act_scale(layer, seed=3)
    blob, _ = cla.pack(layer)
    mod = cla.CompressedLinear(blob, max_M=max(M, 2))
    xs = [make_x(cfg, li, M, K=K) for _ in range(1)]
    r = np.random.default_rng(cfg * 100 + M)
    for t in range(4):
        xs.append((np.asarray(xs[0]).astype(np.float64) * 0 + r.normal(0, 1, (M, K))).astype(np.float16)
                  if layer.x_dtype == "f16" else make_x(cfg, li, M, K=K) ^ np.uint16(t + 1))
    x_static = to_device_x(xs[0], layer.x_dtype)
    y_static = torch.empty((M, N), dtype=torch.float32, device="cuda")
    stream = torch.cuda.Stream()
    say("graph", layer.name, "M", M, path)
    with torch.cuda.stream(stream):
        mod.forward(x_static, out=y_static, path=path)  # warm-up on the capture stream
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        mod.forward(x_static, out=y_static, path=path)
    torch.cuda.synchronize()
    for t, xh in enumerate(xs):
        xd = to_device_x(xh, layer.x_dtype)
        y_eager = mod.forward(xd, path=path).clone()   # an eager forward between replays
        torch.cuda.synchronize()
        x_static.copy_(xd)
        g.replay()
        torch.cuda.synchronize()
        got = y_static.cpu().numpy()
        assert np.array_equal(got, y_eager.cpu().numpy()), f"replay {t} differs from the eager forward"
        check_bound(got.astype(np.float64), layer, xh, what=f"replay {t}")
    mod.close()
