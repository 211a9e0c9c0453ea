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


def header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(cl_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_function():
    names = header_functions()
    assert set(names) == set(cla.EXPORTED_SYMBOLS)
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
    assert L.cl_quant_absmax(fake, 16, 8, 0, 0, fake, fake, None) == -1  # group
    assert L.cl_quant_absmax(None, 16, 8, 4, 0, fake, fake, None) == -1  # NULL factor
