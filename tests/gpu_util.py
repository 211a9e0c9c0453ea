"""Helpers for the GPU tests: run a logical layer through the HIP library, compare with the oracle."""
import numpy as np

import compressed_linear_amd as cla
import oracle


def torch_cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU (run with -m 'not gpu' on CPU)"
    return torch


def to_device_x(x, x_dtype):
    torch = torch_cuda()
    if x_dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x.astype(np.uint16)).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(x.astype(np.float16))).cuda()


def gpu_layer(layer, max_M=32):
    blob, _ = cla.pack(layer)
    return cla.CompressedLinear(blob, max_M=max_M)


def gpu_forward(layer, x, path="auto", mod=None):
    torch = torch_cuda()
    M = x.shape[0]
    own = mod is None
    if own:
        mod = gpu_layer(layer, max_M=max(M, 1))
    y = mod.forward(to_device_x(x, layer.x_dtype), path=path)
    torch.cuda.synchronize()
    out = y.cpu().numpy().astype(np.float64)
    if own:
        mod.close()
    return out


def check_bound(y, layer, x, rows=None, what=""):
    y_ref, B = oracle.forward_and_bound(layer, x, rows)
    if rows is not None:
        y = y[:, rows]
    err = np.abs(y - y_ref)
    bad = err > B
    ratio = float((err / np.maximum(B, 1e-300)).max(initial=0.0))
    assert not bad.any(), f"{what}: {int(bad.sum())} outputs outside the bound, max err/bound {ratio:.3g}"
    return ratio
