"""Test-only decoder of the packed blob back to logical arrays (numpy, CPU).

Written from the layout description of the packer's sections; used to check
that packing is lossless and laid out as documented.  Not used by the library.
"""
import numpy as np

from compressed_linear_amd import blob_header


def _sec(blob, h, name, dtype=np.uint8):
    off, ln = h["sections"][name]
    return np.frombuffer(blob[off:off + ln].tobytes(), dtype=dtype)


def unpack(blob):
    h = blob_header(blob)
    K, N, T, C = h["K"], h["N"], h["n_tiles"], h["chunks"]
    Npad = T * 64
    dense_kind = ["lut3", "lut4", "int4", "int8"][h["dense"]]
    mask = ["none", "2:4", "bitmap"][h["mask"]]
    out = {"K": K, "N": N, "dense": dense_kind, "mask": mask}

    def tiled(name, cb):
        """Row-major chunk stream -> [Npad, C * cb] bytes."""
        return _sec(blob, h, name)[: Npad * C * cb].reshape(Npad, C * cb)

    if dense_kind in ("lut3", "lut4"):
        rows = tiled("dense", 16).view(np.uint32)  # [Npad, C*4]
        if dense_kind == "lut3":
            w = rows.astype(np.uint64)
            b = [(w >> (8 * i)) & 0xFF for i in range(4)]
            pairs = [bi >> 2 for bi in b]
            pairs.append((b[0] & 3) | ((b[1] & 3) << 2) | ((b[2] & 3) << 4))
            assert ((b[3] & 3) == 0).all()
            codes = np.zeros((Npad, C * 40), np.uint8)
            for j, p in enumerate(pairs):
                for half in range(2):
                    kk = np.arange(C * 4)[:, None] * 10 + 2 * j + half
                    codes[:, kk[:, 0]] = ((p >> (3 * half)) & 7).astype(np.uint8)
        else:
            # byte b of a word: pair p = code(2b) | code(2b+1) << 4, rotated left by 2
            codes = np.zeros((Npad, C * 32), np.uint8)
            for b in range(4):
                byte = (rows >> (8 * b)) & 0xFF
                pr = ((byte >> 2) | (byte << 6)) & 0xFF
                codes[:, 2 * b::8] = (pr & 0xF).astype(np.uint8)
                codes[:, 2 * b + 1::8] = (pr >> 4).astype(np.uint8)
        out["codes"] = codes[:N, :K]
        nb = 8 if dense_kind == "lut3" else 16
        out["lut"] = _sec(blob, h, "table", np.uint16).reshape(Npad, nb)[:N].view(np.float16)
    else:
        out["row_scale"] = _sec(blob, h, "table", np.uint16)[:N].view(np.float16)
        if dense_kind == "int4" and mask == "none":
            w = tiled("dense", 16).view(np.uint32)
            q = np.zeros((Npad, C * 32), np.int16)
            for j in range(4):
                q[:, 2 * j::8] = ((w >> (4 * j)) & 0xF).astype(np.int16) - 8
                q[:, 2 * j + 1::8] = ((w >> (16 + 4 * j)) & 0xF).astype(np.int16) - 8
            out["qvals"] = q[:N, :K].astype(np.int8)
        elif dense_kind == "int4":
            w = tiled("dense", 16).view(np.uint32)   # [Npad, C*4]
            m = tiled("meta", 8).view(np.uint32)     # [Npad, C*2]
            q = np.zeros((Npad, C * 64), np.int16)
            keep = np.zeros((Npad, C * 64), np.uint8)
            for c in range(C):
                for g in range(16):
                    wv = w[:, 4 * c + g // 4]
                    nib = (m[:, 2 * c + g // 8] >> (4 * (g % 8))) & 0xF
                    i0, i1 = nib & 3, nib >> 2
                    v0 = ((wv >> (4 * (g % 4))) & 0xF).astype(np.int16) - 8
                    v1 = ((wv >> (16 + 4 * (g % 4))) & 0xF).astype(np.int16) - 8
                    base = 64 * c + 4 * g
                    r = np.arange(Npad)
                    q[r, base + i0] = v0
                    q[r, base + i1] = v1
                    keep[r, base + i0] = 1
                    keep[r, base + i1] = 1
            out["qvals"] = q[:N, :K].astype(np.int8)
            out["keep"] = keep[:N, :K]
        elif mask == "none":
            b = tiled("dense", 16)
            out["qvals"] = (b[:N, :K].astype(np.int16) - 128).astype(np.int8)
        else:
            bm = tiled("meta", 16).view(np.uint32)  # [Npad, C*4]
            bits = ((bm[:, :, None] >> np.arange(32)[None, None, :]) & 1).reshape(Npad, C * 128).astype(np.uint8)
            keep = bits[:N, :K]
            nzoff = _sec(blob, h, "nzoff", np.int32)
            nz = _sec(blob, h, "dense", np.int8)
            q = np.zeros((N, K), np.int8)
            for n in range(N):
                ks = np.flatnonzero(keep[n])
                q[n, ks] = nz[nzoff[n]:nzoff[n] + ks.size]
            out["qvals"], out["keep"] = q, keep
    if h["nnz"]:
        out["csr_row_ptr"] = _sec(blob, h, "rowptr", np.int32)
        out["csr_col"] = _sec(blob, h, "col", np.int32)
        out["csr_val"] = _sec(blob, h, "val", np.uint16).view(np.float16)
    if h["lr"]:
        r, g = h["rank"], max(h["group"], 1)
        # factors are stored transposed: L^T [r][K], R^T [Npad][r]
        if h["lr"] == 3:
            hk, hr = (K + 1) // 2, (r + 1) // 2
            Lb = _sec(blob, h, "L").reshape(r, hk)
            LqT = np.stack([(Lb & 0xF), (Lb >> 4)], axis=2).reshape(r, 2 * hk)[:, :K].astype(np.int16) - 8
            Rb = _sec(blob, h, "R").reshape(Npad, hr)
            RqT = np.stack([(Rb & 0xF), (Rb >> 4)], axis=2).reshape(Npad, 2 * hr)[:N, :r].astype(np.int16) - 8
            out["L"], out["R"] = LqT.T.astype(np.int8), RqT.T.astype(np.int8)
            gk, gr = -(-K // g), -(-r // g)
            out["L_scale"] = _sec(blob, h, "Lscale", np.uint16).reshape(r, gk).T.view(np.float16)
            out["R_scale"] = _sec(blob, h, "Rscale", np.uint16).reshape(Npad, gr)[:N].T.view(np.float16)
        else:
            out["L"] = _sec(blob, h, "L", np.uint16).reshape(r, K).T
            out["R"] = _sec(blob, h, "R", np.uint16).reshape(Npad, r)[:N].T
    if h["n_xscale"]:
        # dense fp16 factor per input channel, 1 (0x3C00) where unscaled
        xs = _sec(blob, h, "xscale", np.uint16)
        assert xs.size == K
        ch = np.flatnonzero(xs != 0x3C00).astype(np.int32)
        out["xscale_dense"] = xs.view(np.float16)
        out["xscale_ch"], out["xscale"] = ch, xs[ch].view(np.float16)
    return h, out
