"""The C ABI: exported symbols, struct layouts, and host-side error handling (no GPU)."""
import ctypes
import os
import re
import subprocess
import tempfile

import numpy as np
import pytest

import compressed_linear_amd as cla

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "compressed_linear.h")
PROBE_HEADER = os.path.join(ROOT, "include", "cl_probe.h")


def header_functions(path=HEADER):
    src = open(path).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(cl_[a-z_0-9]+)\s*\(", src)))


def test_library_exports_every_declared_function():
    assert set(header_functions()) == set(cla.EXPORTED_SYMBOLS)
    assert set(header_functions(PROBE_HEADER)) == set(cla.PROBE_SYMBOLS)
    names = header_functions() + header_functions(PROBE_HEADER)
    L = cla.lib()
    for n in names:
        assert hasattr(L, n), n
    nm = subprocess.run(["nm", "-D", "--defined-only", cla.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (cl_\w+)", nm))
    assert set(names) <= exported


def test_struct_layouts_match_header(tmp_path):
    prog = tmp_path / "sz.c"
    prog.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "compressed_linear.h"\n'
                    'int main(void){printf("%zu %zu %zu %zu %zu %zu\\n", sizeof(cl_layer_desc), sizeof(cl_bytes),'
                    ' sizeof(cl_blob_header), offsetof(cl_layer_desc, x_dtype), offsetof(cl_blob_header, acct),'
                    ' offsetof(cl_blob_header, off));return 0;}\n')
    exe = tmp_path / "sz"
    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), str(prog), "-o", str(exe)], check=True)
    got = [int(v) for v in subprocess.run([str(exe)], capture_output=True, text=True).stdout.split()]
    want = [ctypes.sizeof(cla.cl_layer_desc), ctypes.sizeof(cla.cl_bytes), ctypes.sizeof(cla.cl_blob_header),
            cla.cl_layer_desc.x_dtype.offset, cla.cl_blob_header.acct.offset, cla.cl_blob_header.off.offset]
    assert got == want


def test_host_errors_without_gpu():
    L = cla.lib()
    y = ctypes.c_float()
    assert L.cl_forward(None, 1, None, None, None) == -1
    assert b"handle" in L.cl_last_error()
    assert L.cl_debug_dequant(None, None, None, None, None, None) == -1
    assert L.cl_destroy(None) == 0
    assert L.cl_set_wait_limit(None, 0, 1) == -1
    assert L.cl_device_bytes(None, 1) == 0
    h = ctypes.c_void_p()
    assert L.cl_create(None, None, 0, 1, None, ctypes.byref(h)) == -1
    junk = np.zeros(4096, np.uint8)
    assert L.cl_create(junk.ctypes.data, None, 0, 1, None, ctypes.byref(h)) == -1
    assert b"magic" in L.cl_last_error()


def test_packer_entry_points_validate_on_the_host():
    # argument errors come back before any device work (no GPU needed)
    L = cla.lib()
    fake = ctypes.c_void_p(256)  # never dereferenced: validation fails first
    assert L.cl_fit_lut_work_bytes(0, 5) == 0 and L.cl_fit_lut_work_bytes(4, 4) > 0
    assert L.cl_fit_lut(fake, 4, 64, 5, 1, 10, fake, fake, fake, fake, fake, fake, None, None) == -1  # bits
    assert b"bits" in L.cl_last_error()
    assert L.cl_fit_lut(fake, 4, 40000, 3, 1, 10, fake, fake, fake, fake, fake, fake, None, None) == -5  # K too big
    assert L.cl_fit_lut(fake, 4, 64, 3, 10 ** 6, 10, fake, fake, fake, fake, fake, fake, None, None) == -1  # n_out
    assert L.cl_fit_lut(fake, 4, 64, 4, 1, 0, fake, fake, fake, fake, fake, fake, None, None) == -1  # max_iter
    assert L.cl_fit_lut(None, 4, 64, 4, 1, 5, fake, fake, fake, fake, fake, fake, None, None) == -1  # NULL W
    assert L.cl_fit_int(fake, 4, 64, 8, 1, 10, fake, fake, fake, fake, None) == -2  # 2:4 needs int4
    assert L.cl_fit_int(fake, 4, 62, 4, 1, 10, fake, fake, fake, fake, None) == -2  # 2:4 needs K % 4 == 0
    assert L.cl_fit_int(fake, 4, 64, 4, 2, 10, fake, fake, fake, fake, None) == -2  # unstructured needs int8
    assert L.cl_fit_int(fake, 4, 64, 5, 0, 10, fake, fake, fake, fake, None) == -1  # bits
    assert L.cl_fit_int(fake, 4, 64, 4, 0, 0, fake, fake, fake, fake, None) == -1  # grid
    assert L.cl_fit_int(fake, 4, 64, 4, 1, 10, fake, fake, None, fake, None) == -1  # keep required with a mask
    # the fitter without a work buffer: rows beyond its static scratch, before any device work
    assert L.cl_fit_lut_noalloc(fake, 200000, 64, 4, 1, 10, fake, fake, fake, fake, fake, None, None) == -5
    assert b"N <= 130972" in L.cl_last_error()
    assert L.cl_fit_lut_noalloc(fake, 4, 64, 5, 1, 10, fake, fake, fake, fake, fake, None, None) == -1  # bits
    assert L.cl_quant_absmax(fake, 16, 8, 0, 0, fake, fake, None) == -1  # group
    assert L.cl_quant_absmax(None, 16, 8, 4, 0, fake, fake, None) == -1  # NULL factor


def _blob_of(layer):
    blob, _ = cla.pack(layer)
    return blob.copy()


def _section(blob, name, dtype):
    off, ln = cla.blob_header(blob)["sections"][name]
    return blob[off:off + ln].view(dtype)


def _device_bytes(blob, max_M=1):
    L = cla.lib()
    n = L.cl_device_bytes(blob.ctypes.data, max_M)
    return n, L.cl_last_error().decode()


def _set_header(blob, field, value, index=None):
    h = cla.cl_blob_header.from_buffer(blob)
    if index is None:
        setattr(h, field, value)
    else:
        getattr(h, field)[index] = value
    return blob


def test_corrupt_blobs_are_rejected_on_the_host():
    # cl_create and the kernels trust a blob only after check_blob; cl_device_bytes runs the
    # same check without a GPU and returns 0 (with the reason in cl_last_error) for a bad blob
    from synth.layers import make_layer
    good = _blob_of(make_layer(1, 0, K=200, N=70))
    assert _device_bytes(good)[0] > 0
    nnz = int(cla.blob_header(good)["nnz"])
    assert nnz > 3

    def bad(mutate, word):
        b = good.copy()
        mutate(b)
        n, msg = _device_bytes(b)
        assert n == 0 and word in msg, msg

    bad(lambda b: _section(b, "rowptr", np.int32).__setitem__(5, 10 ** 6), "CSR")  # decreasing after row 5
    bad(lambda b: _section(b, "rowptr", np.int32).__setitem__(-1, nnz - 1), "CSR")  # does not end at nnz
    bad(lambda b: _section(b, "col", np.int32).__setitem__(0, 200), "CSR")  # column == K
    bad(lambda b: _section(b, "col", np.int32).__setitem__(0, -1), "CSR")
    rp = _section(good, "rowptr", np.int32)
    row = int(np.argmax(np.diff(rp) >= 2))
    bad(lambda b: _section(b, "col", np.int32).__setitem__(rp[row] + 1, _section(b, "col", np.int32)[rp[row]]),
        "increasing")  # a repeated column
    # section bounds: an offset that would wrap, a length that disagrees with the header
    s_col = cla.SECTIONS.index("col")
    bad(lambda b: _set_header(b, "off", (1 << 64) - 256, s_col), "outside")
    bad(lambda b: _set_header(b, "len", 4 * nnz - 4, s_col), "implies")
    bad(lambda b: _set_header(b, "total_bytes", 1024), "outside")
    # header fields that disagree with each other
    bad(lambda b: _set_header(b, "chunks", 3), "format")
    bad(lambda b: _set_header(b, "rank", 8), "low-rank")
    bad(lambda b: _set_header(b, "nnz", -1), "nnz")
    # bitmap: a row's offsets too short for its kept values, keep bits on a padding row
    gb = _blob_of(make_layer(4, 0, K=256, N=70, M_for_clamp=2))
    assert _device_bytes(gb)[0] > 0
    b = gb.copy()
    nzo = _section(b, "nzoff", np.int32)
    nzo[1] = nzo[0]
    n, msg = _device_bytes(b)
    assert n == 0 and "bitmap" in msg, msg
    b = gb.copy()
    meta = _section(b, "meta", np.uint32).reshape(128, -1)  # Npad = 128 rows of keep bits
    meta[100, 0] = 1
    n, msg = _device_bytes(b)
    assert n == 0 and "padding" in msg, msg


def test_buffers_of_2_gib_are_refused():
    # the kernels address every buffer through a 32-bit range: no section or workspace
    # buffer may reach 2 GiB (CL_ESIZE), checked before any array is read
    L = cla.lib()
    d = cla.cl_layer_desc()
    d.K, d.N = 1 << 24, 1 << 13
    d.dense = 0
    d.codes = 256  # never dereferenced: the size check comes first
    d.lut = 256
    size = ctypes.c_size_t(0)
    assert L.cl_pack(ctypes.byref(d), None, ctypes.byref(size), None) == -5
    assert b"2^31" in L.cl_last_error()
    from synth.layers import make_layer
    blob = _blob_of(make_layer(1, 0, K=4096, N=64))
    assert L.cl_device_bytes(blob.ctypes.data, 1) > 0
    assert L.cl_device_bytes(blob.ctypes.data, 1 << 18) == 0  # activations of 2^18 rows: 2 GiB
    assert b"2 GiB" in L.cl_last_error()


def test_fit_lowrank_host_checks():
    # argument errors are reported before any device work (no GPU needed)
    L = cla.lib()
    assert L.cl_fit_lowrank(None, 10, 10, 2, 4, 2, 0, 1, 1, None, None) == -1          # E NULL
    assert L.cl_fit_lowrank(1, 10, 10, 0, 4, 2, 0, 1, 1, None, None) == -1             # rank 0
    assert L.cl_fit_lowrank(1, 10, 10, 513, 4, 2, 0, 1, 1, None, None) == -1           # rank above 512
    assert L.cl_fit_lowrank(1, 10, 10, 2, -1, 2, 0, 1, 1, None, None) == -1            # oversample < 0
    assert L.cl_fit_lowrank(1, 10, 10, 2, 4, 101, 0, 1, 1, None, None) == -1           # iters > 100
    assert L.cl_fit_lowrank(1, 1 << 16, 1 << 16, 2, 4, 2, 0, 1, 1, None, None) == -5   # 2^32 elements
