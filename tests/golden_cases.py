"""Load the hand-derived fixtures under tests/golden/ as logical layers."""
import glob
import json
import os

import numpy as np

from synth.layers import LogicalLayer

GOLDEN_DIR = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def golden_names():
    return sorted(os.path.basename(p)[:-5] for p in glob.glob(os.path.join(GOLDEN_DIR, "*.json")))


def load_golden(name):
    with open(os.path.join(GOLDEN_DIR, name + ".json")) as f:
        g = json.load(f)
    K, N = g["K"], g["N"]
    kw = dict(K=K, N=N, dense=g["dense"], mask=g.get("mask", "none"), x_dtype=g["x_dtype"], name=name)
    if "lut" in g:
        kw["lut"] = np.array(g["lut"], dtype=np.float16)
        kw["codes"] = np.array(g["codes"], dtype=np.uint8)
    if "qvals" in g:
        kw["qvals"] = np.array(g["qvals"], dtype=np.int8)
        kw["row_scale"] = np.array(g["row_scale"], dtype=np.float16)
    if "keep" in g:
        kw["keep"] = np.array(g["keep"], dtype=np.uint8)
    if "csr_row_ptr" in g:
        kw["csr_row_ptr"] = np.array(g["csr_row_ptr"], dtype=np.int32)
        kw["csr_col"] = np.array(g["csr_col"], dtype=np.int32)
        kw["csr_val"] = np.array(g["csr_val"], dtype=np.float16)
    if "act_clamp" in g:
        kw["act_clamp"] = np.float16(g["act_clamp"])
    if "xscale_ch" in g:
        kw["xscale_ch"] = np.array(g["xscale_ch"], dtype=np.int32)
        kw["xscale"] = np.array(g["xscale"], dtype=np.float16)
        assert np.array_equal(kw["xscale"].astype(np.float64), np.array(g["xscale"])), "factor not exact in fp16"
    lr = g.get("lr", "none")
    kw["lr"] = lr
    if lr != "none":
        kw["rank"] = g["rank"]
        kw["group"] = g.get("group", 128)
        if lr == "int4":
            kw["L"] = np.array(g["L"], dtype=np.int8)
            kw["R"] = np.array(g["R"], dtype=np.int8)
            kw["L_scale"] = np.array(g["L_scale"], dtype=np.float16)
            kw["R_scale"] = np.array(g["R_scale"], dtype=np.float16)
        elif lr == "bf16":
            kw["L"] = np.array(g["L_bf16_bits"], dtype=np.uint16)
            kw["R"] = np.array(g["R_bf16_bits"], dtype=np.uint16)
        else:
            kw["L"] = np.array(g["L"], dtype=np.float16)
            kw["R"] = np.array(g["R"], dtype=np.float16)
    layer = LogicalLayer(**kw)
    if g["x_dtype"] == "bf16":
        x = np.array(g["x_bf16_bits"], dtype=np.uint16)
    else:
        x = np.array(g["x"], dtype=np.float16)
    return layer, x, np.array(g["expected_y"], dtype=np.float64), g
