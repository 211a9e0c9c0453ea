"""Python binding of the MI355X compressed linear layer library.

Argument marshalling only: every step of the forward runs in the HIP
library `libcompressed_linear.so` (built in-tree by
`python -m compressed_linear_amd.build`).  PyTorch supplies device memory and
streams.  Importing works without a GPU; constructing a `CompressedLinear`
needs one.  A missing library raises at first use -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

__all__ = ["ClError", "lib", "pack", "blob_header", "CompressedLinear", "fit_lut", "fit_int", "quant_absmax", "LIB_PATH",
           "EXPORTED_SYMBOLS", "PROBE_SYMBOLS"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libcompressed_linear.so")

EXPORTED_SYMBOLS = [
    "cl_pack", "cl_device_bytes", "cl_create", "cl_forward", "cl_forward_path",
    "cl_debug_dequant", "cl_destroy", "cl_last_error", "cl_fit_lut_work_bytes", "cl_fit_lut",
    "cl_fit_int", "cl_quant_absmax", "cl_set_wait_limit", "cl_fit_lut_noalloc", "cl_fit_lowrank",
]

# measurement aids of the benchmark (include/cl_probe.h), exported by the same library
PROBE_SYMBOLS = ["cl_probe_read", "cl_probe_read_sink_words", "cl_probe_empty"]

DENSE = {"lut3": 0, "lut4": 1, "int4": 2, "int8": 3}
MASK = {"none": 0, "2:4": 1, "bitmap": 2}
LR = {"none": 0, "fp16": 1, "bf16": 2, "int4": 3}
ACT = {"f16": 0, "bf16": 1}
PATH = {"auto": 0, "decode": 1, "prefill": 2, "decode_valu": 3, "decode_mfma": 4, "decode_stream": 5}
STATUS = {0: "CL_OK", -1: "CL_EINVAL", -2: "CL_EUNSUPPORTED", -3: "CL_ENOMEM", -4: "CL_EHIP", -5: "CL_ESIZE"}
SECTIONS = ["dense", "table", "meta", "nzoff", "rowptr", "col", "val", "L", "R", "Lscale", "Rscale", "xscale"]
SEC_COUNT = 16


class ClError(RuntimeError):
    def __init__(self, status: int, where: str, msg: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)}: {msg}")


class cl_layer_desc(ctypes.Structure):
    _fields_ = [
        ("K", ctypes.c_int32), ("N", ctypes.c_int32), ("dense", ctypes.c_int32), ("mask", ctypes.c_int32),
        ("codes", ctypes.c_void_p), ("lut", ctypes.c_void_p), ("qvals", ctypes.c_void_p),
        ("row_scale", ctypes.c_void_p), ("keep", ctypes.c_void_p),
        ("nnz", ctypes.c_int64), ("csr_row_ptr", ctypes.c_void_p), ("csr_col", ctypes.c_void_p),
        ("csr_val", ctypes.c_void_p),
        ("lr", ctypes.c_int32), ("rank", ctypes.c_int32), ("group", ctypes.c_int32),
        ("L", ctypes.c_void_p), ("R", ctypes.c_void_p), ("L_scale", ctypes.c_void_p), ("R_scale", ctypes.c_void_p),
        ("has_clamp", ctypes.c_int32), ("act_clamp", ctypes.c_uint16), ("reserved0", ctypes.c_uint16),
        ("x_dtype", ctypes.c_int32),
        ("n_xscale", ctypes.c_int32), ("xscale_ch", ctypes.c_void_p), ("xscale", ctypes.c_void_p),
    ]


class cl_bytes(ctypes.Structure):
    _fields_ = [(n, ctypes.c_uint64) for n in
                ("codes", "lut_or_scale", "mask_meta", "csr", "lowrank", "act_scale", "total", "device_padding")]


class cl_blob_header(ctypes.Structure):
    _fields_ = [
        ("magic", ctypes.c_uint32), ("version", ctypes.c_uint32),
        ("K", ctypes.c_int32), ("N", ctypes.c_int32), ("dense", ctypes.c_int32), ("mask", ctypes.c_int32),
        ("lr", ctypes.c_int32), ("rank", ctypes.c_int32), ("group", ctypes.c_int32), ("x_dtype", ctypes.c_int32),
        ("has_clamp", ctypes.c_int32), ("act_clamp", ctypes.c_uint16), ("reserved0", ctypes.c_uint16),
        ("n_tiles", ctypes.c_int32), ("chunks", ctypes.c_int32), ("span", ctypes.c_int32),
        ("meta_chunk_bytes", ctypes.c_int32), ("nnz", ctypes.c_int64), ("total_bytes", ctypes.c_uint64),
        ("off", ctypes.c_uint64 * SEC_COUNT), ("len", ctypes.c_uint64 * SEC_COUNT),
        ("acct", cl_bytes), ("n_xscale", ctypes.c_int32), ("reserved", ctypes.c_uint8 * 60),
    ]


_lib = None


def lib():
    """The loaded HIP library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m compressed_linear_amd.build`")
        # torch's HIP runtime has the same soname as the system one the library
        # links against: load torch first, so that the library binds to the
        # runtime that owns torch's device memory and streams (loading the
        # library first makes torch bind to the system runtime instead, and
        # the two then disagree about the devices)
        import torch  # noqa: F401
        L = ctypes.CDLL(LIB_PATH)
        L.cl_pack.argtypes = [ctypes.POINTER(cl_layer_desc), ctypes.c_void_p, ctypes.POINTER(ctypes.c_size_t),
                              ctypes.POINTER(cl_bytes)]
        L.cl_pack.restype = ctypes.c_int
        L.cl_device_bytes.argtypes = [ctypes.c_void_p, ctypes.c_int32]
        L.cl_device_bytes.restype = ctypes.c_size_t
        L.cl_create.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_void_p,
                                ctypes.POINTER(ctypes.c_void_p)]
        L.cl_create.restype = ctypes.c_int
        L.cl_forward.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        L.cl_forward.restype = ctypes.c_int
        L.cl_forward_path.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                                      ctypes.c_void_p, ctypes.c_int32]
        L.cl_forward_path.restype = ctypes.c_int
        L.cl_debug_dequant.argtypes = [ctypes.c_void_p] + [ctypes.c_void_p] * 5
        L.cl_debug_dequant.restype = ctypes.c_int
        L.cl_destroy.argtypes = [ctypes.c_void_p]
        L.cl_destroy.restype = ctypes.c_int
        L.cl_last_error.argtypes = []
        L.cl_last_error.restype = ctypes.c_char_p
        L.cl_fit_lut_work_bytes.argtypes = [ctypes.c_int32, ctypes.c_int32]
        L.cl_fit_lut_work_bytes.restype = ctypes.c_size_t
        L.cl_fit_lut.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int64,
                                 ctypes.c_int32] + [ctypes.c_void_p] * 7 + [ctypes.POINTER(ctypes.c_int64)]
        L.cl_fit_lut.restype = ctypes.c_int
        L.cl_fit_int.argtypes = [ctypes.c_void_p] + [ctypes.c_int32] * 5 + [ctypes.c_void_p] * 5
        L.cl_fit_int.restype = ctypes.c_int
        L.cl_quant_absmax.argtypes = [ctypes.c_void_p] + [ctypes.c_int32] * 4 + [ctypes.c_void_p] * 3
        L.cl_quant_absmax.restype = ctypes.c_int
        L.cl_fit_lowrank.argtypes = ([ctypes.c_void_p] + [ctypes.c_int32] * 5 + [ctypes.c_uint64] +
                                     [ctypes.c_void_p] * 4)
        L.cl_fit_lowrank.restype = ctypes.c_int
        L.cl_fit_lut_noalloc.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                         ctypes.c_int64, ctypes.c_int32] + [ctypes.c_void_p] * 6 + \
            [ctypes.POINTER(ctypes.c_int64)]
        L.cl_fit_lut_noalloc.restype = ctypes.c_int
        L.cl_set_wait_limit.argtypes = [ctypes.c_void_p, ctypes.c_uint32, ctypes.c_int32]
        L.cl_set_wait_limit.restype = ctypes.c_int
        L.cl_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]
        L.cl_probe_read.restype = ctypes.c_int
        L.cl_probe_read_sink_words.argtypes = [ctypes.c_size_t]
        L.cl_probe_read_sink_words.restype = ctypes.c_size_t
        L.cl_probe_empty.argtypes = [ctypes.c_void_p]
        L.cl_probe_empty.restype = ctypes.c_int
        _lib = L
    return _lib


def _check(st: int, where: str):
    if st != 0:
        raise ClError(st, where, lib().cl_last_error().decode(errors="replace"))


def _ptr(a: Optional[np.ndarray], dtype, keep: list):
    if a is None:
        return None
    arr = np.ascontiguousarray(a, dtype=dtype)
    keep.append(arr)
    return arr.ctypes.data


def _u16(a, keep):
    """fp16 arrays -> their bits; uint16 arrays (bf16 bits) pass through."""
    if a is None:
        return None
    a = np.asarray(a)
    if a.dtype == np.float16:
        a = a.view(np.uint16)
    return _ptr(a, np.uint16, keep)


def _desc(layer, keep: list) -> cl_layer_desc:
    d = cl_layer_desc()
    d.K, d.N = int(layer.K), int(layer.N)
    d.dense = DENSE[layer.dense]
    d.mask = MASK[getattr(layer, "mask", "none")]
    d.codes = _ptr(getattr(layer, "codes", None), np.uint8, keep)
    d.lut = _u16(getattr(layer, "lut", None), keep)
    d.qvals = _ptr(getattr(layer, "qvals", None), np.int8, keep)
    d.row_scale = _u16(getattr(layer, "row_scale", None), keep)
    d.keep = _ptr(getattr(layer, "keep", None), np.uint8, keep)
    col = getattr(layer, "csr_col", None)
    d.nnz = 0 if col is None else int(np.asarray(col).size)
    if d.nnz:
        d.csr_row_ptr = _ptr(layer.csr_row_ptr, np.int32, keep)
        d.csr_col = _ptr(layer.csr_col, np.int32, keep)
        d.csr_val = _u16(layer.csr_val, keep)
    lr = getattr(layer, "lr", "none")
    rank = int(getattr(layer, "rank", 0) or 0)
    d.lr = LR[lr] if rank > 0 else 0
    d.rank = rank if lr != "none" else 0
    d.group = int(getattr(layer, "group", 128) or 128)
    if d.lr == LR["int4"]:
        d.L = _ptr(layer.L, np.int8, keep)
        d.R = _ptr(layer.R, np.int8, keep)
        d.L_scale = _u16(layer.L_scale, keep)
        d.R_scale = _u16(layer.R_scale, keep)
    elif d.lr:
        d.L = _u16(layer.L, keep)
        d.R = _u16(layer.R, keep)
    c = getattr(layer, "act_clamp", None)
    d.has_clamp = 0 if c is None else 1
    d.act_clamp = 0 if c is None else int(np.array(c, dtype=np.float16).view(np.uint16))
    d.x_dtype = ACT[getattr(layer, "x_dtype", "f16")]
    ch = getattr(layer, "xscale_ch", None)
    if ch is not None and len(ch):
        d.n_xscale = int(len(ch))
        d.xscale_ch = _ptr(ch, np.int32, keep)
        d.xscale = _u16(layer.xscale, keep)
    return d


def pack(layer):
    """Validate and pack a logical layer (any object with the documented attributes).

    Returns (blob, acct): blob is a 16-byte aligned uint8 numpy array, acct the
    canonical byte accounting as a dict.
    """
    keep: list = []
    d = _desc(layer, keep)
    size = ctypes.c_size_t(0)
    acct = cl_bytes()
    _check(lib().cl_pack(ctypes.byref(d), None, ctypes.byref(size), ctypes.byref(acct)), "cl_pack(size)")
    raw = np.zeros(size.value + 64, dtype=np.uint8)
    off = (-raw.ctypes.data) % 64
    blob = raw[off:off + size.value]
    _check(lib().cl_pack(ctypes.byref(d), blob.ctypes.data, ctypes.byref(size), ctypes.byref(acct)), "cl_pack")
    return blob, {f: int(getattr(acct, f)) for f, _ in cl_bytes._fields_}


def blob_header(blob: np.ndarray) -> dict:
    h = cl_blob_header.from_buffer_copy(bytes(blob[: ctypes.sizeof(cl_blob_header)]))
    out = {f: getattr(h, f) for f, _ in cl_blob_header._fields_ if f not in ("off", "len", "acct", "reserved")}
    out["sections"] = {SECTIONS[i]: (int(h.off[i]), int(h.len[i])) for i in range(len(SECTIONS)) if h.len[i]}
    out["acct"] = {f: int(getattr(h.acct, f)) for f, _ in cl_bytes._fields_}
    return out


class CompressedLinear:
    """A packed layer resident on one GPU; forward(x) -> y (fp32).

    Device memory (packed layer + workspace) is one torch uint8 tensor.  Calls
    run on torch's current stream.  One forward at a time per instance.
    """

    def __init__(self, blob: np.ndarray, max_M: int = 32, device=None):
        import torch

        self._torch = torch
        dv = torch.device(device if device is not None else "cuda")
        if dv.index is None:
            dv = torch.device("cuda", torch.cuda.current_device())
        self.device = dv
        hdr = blob_header(blob)
        self.K, self.N = hdr["K"], hdr["N"]
        self.rank = hdr["rank"] if hdr["lr"] else 0
        self.x_dtype = torch.bfloat16 if hdr["x_dtype"] == 1 else torch.float16
        self.max_M = int(max_M)
        self.acct = hdr["acct"]
        self._blob = np.ascontiguousarray(blob)
        nbytes = lib().cl_device_bytes(self._blob.ctypes.data, self.max_M)
        if nbytes == 0:
            raise ClError(-1, "cl_device_bytes", "malformed blob or max_M")
        self.dev_bytes = int(nbytes)
        with torch.cuda.device(self.device):
            self._buf = torch.empty(self.dev_bytes + 256, dtype=torch.uint8, device=self.device)
            base = self._buf.data_ptr()
            self._base = base + ((-base) % 256)
            h = ctypes.c_void_p()
            st = lib().cl_create(self._blob.ctypes.data, self._base, self.dev_bytes, self.max_M,
                                 torch.cuda.current_stream(self.device).cuda_stream, ctypes.byref(h))
            _check(st, "cl_create")
        self._h = h

    def forward(self, x, out=None, path: str = "auto"):
        torch = self._torch
        if x.dim() == 1:
            x = x.unsqueeze(0)
        if x.dtype != self.x_dtype or x.device != self.device or x.shape[-1] != self.K:
            raise ValueError(f"x must be {self.x_dtype} [M, {self.K}] on {self.device}")
        x = x.contiguous()
        M = x.shape[0]
        y = out if out is not None else torch.empty((M, self.N), dtype=torch.float32, device=self.device)
        st = lib().cl_forward_path(self._h, M, x.data_ptr(), y.data_ptr(),
                                   torch.cuda.current_stream(self.device).cuda_stream, PATH[path])
        _check(st, "cl_forward")
        return y

    __call__ = forward

    def forward_ptr(self, M: int, x_ptr: int, y_ptr: int, stream: int, path: str = "auto"):
        """Raw-pointer forward (no allocation, no checks beyond the library's)."""
        _check(lib().cl_forward_path(self._h, M, x_ptr, y_ptr, stream, PATH[path]), "cl_forward")

    def debug_dequant(self):
        torch = self._torch
        D16 = torch.empty((self.N, self.K), dtype=torch.float16, device=self.device)
        S16 = torch.empty((self.N, self.K), dtype=torch.float16, device=self.device)
        L32 = R32 = None
        if self.rank:
            L32 = torch.empty((self.K, self.rank), dtype=torch.float32, device=self.device)
            R32 = torch.empty((self.rank, self.N), dtype=torch.float32, device=self.device)
        st = lib().cl_debug_dequant(self._h, D16.data_ptr(), S16.data_ptr(),
                                    None if L32 is None else L32.data_ptr(),
                                    None if R32 is None else R32.data_ptr(),
                                    torch.cuda.current_stream(self.device).cuda_stream)
        _check(st, "cl_debug_dequant")
        return D16, S16, L32, R32

    def set_wait_limit(self, max_polls: int = 1 << 20, withhold: bool = False):
        """Test support (cl_set_wait_limit): the bound of the in-launch wait for
        x' L, and a switch that withholds its publication."""
        _check(lib().cl_set_wait_limit(self._h, int(max_polls), 1 if withhold else 0), "cl_set_wait_limit")

    def close(self):
        if getattr(self, "_h", None):
            lib().cl_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:  # noqa: BLE001 -- interpreter shutdown
            pass


def fit_lut(W, bits: int, n_out: int, max_iter: int = 50, stats: Optional[dict] = None):
    """Data-free LUT packing on the GPU (cl_fit_lut): W is a torch fp16 [N, K]
    tensor on a ROCm device.  Returns device tensors (codes uint8 [N, K], lut
    fp16 [N, 2^bits], row_ptr int32 [N+1], col int32 [n_out], val fp16 [n_out]);
    `stats`, if given, receives the Lloyd iterations run (summed over rows)."""
    import torch
    if W.dtype != torch.float16 or W.dim() != 2 or not W.is_cuda:
        raise ValueError("W must be a 2-D float16 tensor on a ROCm device")
    W = W.contiguous()
    N, K = W.shape
    dev = W.device
    codes = torch.empty((N, K), dtype=torch.uint8, device=dev)
    lut = torch.empty((N, 1 << bits), dtype=torch.float16, device=dev)
    row_ptr = torch.empty(N + 1, dtype=torch.int32, device=dev)
    col = torch.empty(max(n_out, 1), dtype=torch.int32, device=dev)
    val = torch.empty(max(n_out, 1), dtype=torch.float16, device=dev)
    work = torch.empty(max(int(lib().cl_fit_lut_work_bytes(N, K)), 8), dtype=torch.uint8, device=dev)
    iters = ctypes.c_int64(0)
    st = lib().cl_fit_lut(W.data_ptr(), N, K, bits, n_out, max_iter, codes.data_ptr(), lut.data_ptr(),
                          row_ptr.data_ptr(), col.data_ptr(), val.data_ptr(), work.data_ptr(),
                          torch.cuda.current_stream(dev).cuda_stream, ctypes.byref(iters))
    _check(st, "cl_fit_lut")
    if stats is not None:
        stats["total_iters"] = int(iters.value)
    return codes, lut, row_ptr, col[:n_out], val[:n_out]


def fit_int(W, bits: int, mask: str = "none", grid: int = 100):
    """Data-free integer packing on the GPU (cl_fit_int): W is a torch fp16 [N, K]
    tensor on a ROCm device; mask 'none', '2:4' (bits 4) or 'bitmap' (bits 8, half
    of each row).  Returns device tensors (qvals int8 [N, K], row_scale fp16 [N],
    keep uint8 [N, K] or None)."""
    import torch
    if W.dtype != torch.float16 or W.dim() != 2 or not W.is_cuda:
        raise ValueError("W must be a 2-D float16 tensor on a ROCm device")
    W = W.contiguous()
    N, K = W.shape
    dev = W.device
    q = torch.empty((N, K), dtype=torch.int8, device=dev)
    s = torch.empty(N, dtype=torch.float16, device=dev)
    keep = None if mask == "none" else torch.empty((N, K), dtype=torch.uint8, device=dev)
    work = torch.empty(8, dtype=torch.uint8, device=dev)
    st = lib().cl_fit_int(W.data_ptr(), N, K, bits, MASK[mask], grid, q.data_ptr(), s.data_ptr(),
                          None if keep is None else keep.data_ptr(), work.data_ptr(),
                          torch.cuda.current_stream(dev).cuda_stream)
    _check(st, "cl_fit_int")
    return q, s, keep


def quant_absmax(F, group: int = 128):
    """AbsMax int4 groups of a factor on the GPU (cl_quant_absmax): F is a torch
    fp16 or bf16 [R, C] tensor on a ROCm device, grouped along R.  Returns device
    tensors (q int8 [R, C], scale fp16 [ceil(R / group), C])."""
    import torch
    if F.dtype not in (torch.float16, torch.bfloat16) or F.dim() != 2 or not F.is_cuda:
        raise ValueError("F must be a 2-D float16 / bfloat16 tensor on a ROCm device")
    F = F.contiguous()
    R, C = F.shape
    q = torch.empty((R, C), dtype=torch.int8, device=F.device)
    sc = torch.empty((-(-R // group), C), dtype=torch.float16, device=F.device)
    st = lib().cl_quant_absmax(F.data_ptr(), R, C, group, 1 if F.dtype == torch.bfloat16 else 0, q.data_ptr(),
                               sc.data_ptr(), torch.cuda.current_stream(F.device).cuda_stream)
    _check(st, "cl_quant_absmax")
    return q, sc


def fit_lowrank(E, rank: int, oversample: int = 16, iters: int = 8, seed: int = 0):
    """Naive-LoRA factors of the residual E = W - W_hat (cl_fit_lowrank): E is a
    torch float32 [N, K] tensor on a ROCm device.  Returns device tensors
    (L fp32 [K, rank], R fp32 [rank, N]) and the singular-value estimates (a
    host numpy array), with (L R)^T close to E's rank-`rank` truncated SVD."""
    import numpy as np
    import torch
    if E.dtype != torch.float32 or E.dim() != 2 or not E.is_cuda:
        raise ValueError("E must be a 2-D float32 tensor on a ROCm device")
    E = E.contiguous()
    N, K = E.shape
    L = torch.empty((K, rank), dtype=torch.float32, device=E.device)
    R = torch.empty((rank, N), dtype=torch.float32, device=E.device)
    sv = np.zeros(rank, dtype=np.float32)
    st = lib().cl_fit_lowrank(E.data_ptr(), N, K, rank, oversample, iters, seed, L.data_ptr(), R.data_ptr(),
                              sv.ctypes.data, torch.cuda.current_stream(E.device).cuda_stream)
    _check(st, "cl_fit_lowrank")
    return L, R, sv
