"""Byte layout of one 128-token cache page (oracle side).

The pages fix what a page holds, not how its bytes are ordered: MixKVQ
("MixKVQ的系统级实现细节": packed low-bit codes, BF16 salient channels, a
residual), PN-Mix ("核心公式", Appendix G: an LSB plane of 8 tokens/byte for
every channel and an upper-2-bit plane of 4 tokens/byte for high channels, the
pair mask stored once as bits), QJL (Algorithm 1 step 2-3: sign bits and the
norm per key) and the KIVI blog packing rule (low bits first, section 3
``pack2``: code i of a row goes to bits 2*(i mod 4) of byte i//4). This module
states the order this library uses, written out independently of the HIP
kernels; both must produce identical bytes.

Conventions used below. A page holds tokens t = 0..127; tile i = t // 16 and
row r = t % 16, so t = 16*i + r.

2-bit block (256 bytes) of an array X[r][i][k] (r < 16, i < 8, k < 8): the
little-endian dword at byte 16*r + 4*w (w < 4) holds, for every tile i, the
code X[r][i][2w] at bits 2i, 2i+1 and the code X[r][i][2w+1] at bits 16+2i,
16+2i+1. So each byte is a run of four codes of one element along the tile
axis, the lower code in the lower bits as in the KIVI ``pack2`` rule, and the
codes of one tile sit at the same bit position in both 16-bit halves of all
four dwords (the decode kernels mask a tile out of the dwords directly).

1-bit block row (8 bytes) of X[r][i][k]: the little-endian dword w' < 2 at
byte 4*w' holds X[r][i][4z + 2w' + h] at bit 16h + 8(i // 4) + 2(i % 4) + z
(z, h < 2), so that tile i's bits sit, like its 2-bit codes, at the
positions 2(i % 4) (+1) of one byte of each 16-bit half.

The value-code region (4096 bytes) holds, for k-step s < 4 and lane group
a < 4, a 2-bit block at 1024*s + 256*a with X[r][u][k] = code of
V[pi(s,a,k)][16*u + r], where pi(s,a,k) = 32*s + 16*(k//4) + 4*a + k%4. The
value-meta region (2048 bytes) holds at 512*s + 128*a + 32*j the f16 scales
of V[pi(s,a,k)] for channel group j (k = 0..7) followed by their offsets.

Status: the byte order is this library's own convention (parity unpinned as
to order; it is pinned only through the pages' bit-order rule and through
round trips in the tests).
"""
from __future__ import annotations

import numpy as np

from .numerics import f16_fraction, rn_f16_meta_bits

PAGE = 128
D = 128
V_CODE_BYTES = 4096
V_META_BYTES = 2048


def _round_up(x, m):
    return (x + m - 1) // m * m


def pi_token(s: int, a: int, k: int) -> int:
    return 32 * s + 16 * (k // 4) + 4 * a + (k % 4)


# --------------------------------------------------------------- blocks
def pack2_block(X) -> np.ndarray:
    X = np.asarray(X, dtype=np.uint32)
    assert X.shape == (16, 8, 8) and X.max(initial=0) <= 3
    out = np.zeros((16, 4), dtype=np.uint32)
    for r in range(16):
        for w in range(4):
            word = 0
            for i in range(8):
                word |= int(X[r, i, 2 * w]) << (2 * i)
                word |= int(X[r, i, 2 * w + 1]) << (16 + 2 * i)
            out[r, w] = word
    return out.astype("<u4").view(np.uint8).reshape(-1)


def unpack2_block(buf) -> np.ndarray:
    words = np.frombuffer(np.asarray(buf, dtype=np.uint8).tobytes(), dtype="<u4").reshape(16, 4)
    X = np.zeros((16, 8, 8), dtype=np.uint8)
    for r in range(16):
        for w in range(4):
            word = int(words[r, w])
            for i in range(8):
                X[r, i, 2 * w] = (word >> (2 * i)) & 3
                X[r, i, 2 * w + 1] = (word >> (16 + 2 * i)) & 3
    return X


def pack1_rows(X) -> np.ndarray:
    """[16][8][8] bits -> 16 rows x 8 bytes."""
    X = np.asarray(X, dtype=np.uint8)
    assert X.shape == (16, 8, 8) and X.max(initial=0) <= 1
    out = np.zeros((16, 2), dtype=np.uint32)
    for r in range(16):
        for w in range(2):
            word = 0
            for i in range(8):
                for z in range(2):
                    for h in range(2):
                        word |= int(X[r, i, 4 * z + 2 * w + h]) << (16 * h + 8 * (i // 4) + 2 * (i % 4) + z)
            out[r, w] = word
    return out.astype("<u4").view(np.uint8).reshape(16, 8)


def unpack1_rows(rows) -> np.ndarray:
    rows = np.asarray(rows, dtype=np.uint8).reshape(16, 8)
    words = np.frombuffer(rows.tobytes(), dtype="<u4").reshape(16, 2)
    X = np.zeros((16, 8, 8), dtype=np.uint8)
    for r in range(16):
        for w in range(2):
            word = int(words[r, w])
            for i in range(8):
                for z in range(2):
                    for h in range(2):
                        X[r, i, 4 * z + 2 * w + h] = (word >> (16 * h + 8 * (i // 4) + 2 * (i % 4) + z)) & 1
    return X


def _frag_X(slot_codes: np.ndarray, f: int) -> np.ndarray:
    """slot_codes [n_slots_padded][128 tokens] -> X[r][i][k] of fragment f."""
    blk = slot_codes[8 * f: 8 * f + 8]            # [8 k][128 t]
    return blk.reshape(8, 8, 16).transpose(2, 1, 0)   # t = 16 i + r -> [r][i][k]


def _X_to_slots(X: np.ndarray) -> np.ndarray:
    return X.transpose(2, 1, 0).reshape(8, 128)


def pack2_region(slot_codes: np.ndarray) -> np.ndarray:
    n = slot_codes.shape[0]
    F = (n + 7) // 8
    padded = np.zeros((8 * F, PAGE), dtype=np.uint8)
    padded[:n] = slot_codes
    return np.concatenate([pack2_block(_frag_X(padded, f)) for f in range(F)]) if F else np.zeros(0, np.uint8)


def unpack2_region(buf, n_slots: int) -> np.ndarray:
    F = (n_slots + 7) // 8
    out = np.zeros((8 * F, PAGE), dtype=np.uint8)
    for f in range(F):
        out[8 * f: 8 * f + 8] = _X_to_slots(unpack2_block(buf[256 * f: 256 * f + 256]))
    return out[:n_slots]


def pack1_region(slot_bits: np.ndarray) -> np.ndarray:
    n = slot_bits.shape[0]
    F = _round_up((n + 7) // 8, 8)                 # whole fragment pairs of 4 lane groups
    padded = np.zeros((8 * F, PAGE), dtype=np.uint8)
    padded[:n] = slot_bits
    out = np.zeros(128 * F, dtype=np.uint8)
    for P in range(F // 8):
        for a in range(4):
            f1, f2 = 4 * (2 * P) + a, 4 * (2 * P + 1) + a
            r1 = pack1_rows(_frag_X(padded, f1))
            r2 = pack1_rows(_frag_X(padded, f2))
            for r in range(16):
                base = 1024 * P + 256 * a + 16 * r
                out[base: base + 8] = r1[r]
                out[base + 8: base + 16] = r2[r]
    return out


def unpack1_region(buf, n_slots: int) -> np.ndarray:
    F = _round_up((n_slots + 7) // 8, 8)
    out = np.zeros((8 * F, PAGE), dtype=np.uint8)
    buf = np.asarray(buf, dtype=np.uint8)
    for P in range(F // 8):
        for a in range(4):
            f1, f2 = 4 * (2 * P) + a, 4 * (2 * P + 1) + a
            r1 = np.zeros((16, 8), np.uint8)
            r2 = np.zeros((16, 8), np.uint8)
            for r in range(16):
                base = 1024 * P + 256 * a + 16 * r
                r1[r] = buf[base: base + 8]
                r2[r] = buf[base + 8: base + 16]
            out[8 * f1: 8 * f1 + 8] = _X_to_slots(unpack1_rows(r1))
            out[8 * f2: 8 * f2 + 8] = _X_to_slots(unpack1_rows(r2))
    return out[:n_slots]


def _u16_bytes(a) -> np.ndarray:
    return np.asarray(a, dtype="<u2").view(np.uint8).reshape(-1)


def _bytes_u16(b) -> np.ndarray:
    return np.frombuffer(np.asarray(b, dtype=np.uint8).tobytes(), dtype="<u2").copy()


# --------------------------------------------------------------- value part
def pack_v(vcodes, vscale, voff) -> np.ndarray:
    """vcodes [128 t][128 ch] 2-bit; vscale/voff [128 t][4] f16 bits."""
    codes = np.zeros(V_CODE_BYTES, np.uint8)
    meta = np.zeros(V_META_BYTES, np.uint8)
    for s in range(4):
        for a in range(4):
            X = np.zeros((16, 8, 8), np.uint8)
            for k in range(8):
                t = pi_token(s, a, k)
                for u in range(8):
                    X[:, u, k] = vcodes[t, 16 * u: 16 * u + 16]
            codes[1024 * s + 256 * a: 1024 * s + 256 * a + 256] = pack2_block(X)
            for j in range(4):
                toks = [pi_token(s, a, k) for k in range(8)]
                base = 512 * s + 128 * a + 32 * j
                meta[base: base + 16] = _u16_bytes(vscale[toks, j])
                meta[base + 16: base + 32] = _u16_bytes(voff[toks, j])
    return np.concatenate([codes, meta])


def unpack_v(buf):
    buf = np.asarray(buf, dtype=np.uint8)
    vcodes = np.zeros((PAGE, D), np.uint8)
    vscale = np.zeros((PAGE, 4), np.uint16)
    voff = np.zeros((PAGE, 4), np.uint16)
    for s in range(4):
        for a in range(4):
            X = unpack2_block(buf[1024 * s + 256 * a: 1024 * s + 256 * a + 256])
            for k in range(8):
                t = pi_token(s, a, k)
                for u in range(8):
                    vcodes[t, 16 * u: 16 * u + 16] = X[:, u, k]
            for j in range(4):
                toks = [pi_token(s, a, k) for k in range(8)]
                base = V_CODE_BYTES + 512 * s + 128 * a + 32 * j
                vscale[toks, j] = _bytes_u16(buf[base: base + 16])
                voff[toks, j] = _bytes_u16(buf[base + 16: base + 32])
    return vcodes, vscale, voff


# --------------------------------------------------------------- MixKVQ
def mixkvq_geometry(n16: int, n4: int):
    n2 = D - n16 - n4
    s4 = _round_up(2 * n4, 8)
    n_slots = s4 + n2
    F = (n_slots + 7) // 8
    off_codes = 256 * n16
    off_meta = off_codes + 256 * F
    off_v = off_meta + 32 * F
    used = off_v + V_CODE_BYTES + V_META_BYTES
    return dict(n2=n2, s4=s4, n_slots=n_slots, F=F, off_codes=off_codes,
                off_meta=off_meta, off_v=off_v, used=used, stride=_round_up(used, 256))


def _times4_f16(bits: int) -> int:
    """binary16 of 4 s (exact unless it overflows to infinity)."""
    if (bits & 0x7C00) == 0x7C00:
        return bits
    return rn_f16_meta_bits(4 * f16_fraction(bits))


def pack_mixkvq_page(n16, n4, perm, kbits, k4, k2, v):
    """Pack one MixKVQ page.

    perm: channel order (BF16 tier, then UINT4, then UINT2).
    kbits: [128 t][128 ch] bf16 bits of K (BF16-tier channels are copied).
    k4 = (codes [n4][128], scale [n4], offset [n4]); k2 likewise for UINT2.
    v = (codes [128][128], scale [128][4], offset [128][4])."""
    g = mixkvq_geometry(n16, n4)
    page = np.zeros(g["stride"], np.uint8)
    for c in range(n16):
        d = int(perm[c])
        col = kbits[:, d].reshape(8, 16).T          # [r][i]
        page[256 * c: 256 * c + 256] = _u16_bytes(col.reshape(-1))
    slots = np.zeros((g["n_slots"], PAGE), np.uint8)
    sc = np.zeros(8 * g["F"], np.uint16)
    of = np.zeros(8 * g["F"], np.uint16)
    c4, s4v, o4v = k4
    for j in range(n4):
        slots[2 * j] = c4[j] & 3
        slots[2 * j + 1] = c4[j] >> 2
        sc[2 * j], of[2 * j] = s4v[j], o4v[j]
        sc[2 * j + 1], of[2 * j + 1] = _times4_f16(int(s4v[j])), 0
    c2, s2v, o2v = k2
    for j in range(g["n2"]):
        slots[g["s4"] + j] = c2[j]
        sc[g["s4"] + j], of[g["s4"] + j] = s2v[j], o2v[j]
    region = pack2_region(slots)
    page[g["off_codes"]: g["off_codes"] + region.size] = region
    for f in range(g["F"]):
        base = g["off_meta"] + 32 * f
        page[base: base + 16] = _u16_bytes(sc[8 * f: 8 * f + 8])
        page[base + 16: base + 32] = _u16_bytes(of[8 * f: 8 * f + 8])
    page[g["off_v"]: g["off_v"] + V_CODE_BYTES + V_META_BYTES] = pack_v(*v)
    return page


def unpack_mixkvq_page(page, n16, n4, perm):
    """Inverse of pack_mixkvq_page. Returns dict with bf16 K columns, the
    per-tier codes/scales/offsets in channel-position order and the V part."""
    g = mixkvq_geometry(n16, n4)
    page = np.asarray(page, np.uint8)
    kbf = np.zeros((n16, PAGE), np.uint16)
    for c in range(n16):
        kbf[c] = _bytes_u16(page[256 * c: 256 * c + 256]).reshape(16, 8).T.reshape(-1)
    slots = unpack2_region(page[g["off_codes"]: g["off_codes"] + 256 * g["F"]], g["n_slots"])
    sc = np.zeros(8 * g["F"], np.uint16)
    of = np.zeros(8 * g["F"], np.uint16)
    for f in range(g["F"]):
        base = g["off_meta"] + 32 * f
        sc[8 * f: 8 * f + 8] = _bytes_u16(page[base: base + 16])
        of[8 * f: 8 * f + 8] = _bytes_u16(page[base + 16: base + 32])
    c4 = (slots[0: 2 * n4: 2] | (slots[1: 2 * n4: 2] << 2)).astype(np.uint8)
    k4 = (c4, sc[0: 2 * n4: 2].copy(), of[0: 2 * n4: 2].copy())
    k4_hi = (sc[1: 2 * n4: 2].copy(), of[1: 2 * n4: 2].copy())
    n2 = g["n2"]
    k2 = (slots[g["s4"]: g["s4"] + n2].copy(), sc[g["s4"]: g["s4"] + n2].copy(),
          of[g["s4"]: g["s4"] + n2].copy())
    v = unpack_v(page[g["off_v"]:])
    return dict(kbf=kbf, k4=k4, k4_hi_meta=k4_hi, k2=k2, v=v,
                pad_codes=slots[2 * n4: g["s4"]].copy())


# --------------------------------------------------------------- PN-Mix
def pnmix_geometry(n_hi: int):
    n_up_frag = (n_hi + 7) // 8
    off_up = 2048
    off_meta = off_up + 256 * n_up_frag
    off_v = off_meta + 512
    used = off_v + V_CODE_BYTES + V_META_BYTES
    return dict(off_up=off_up, off_meta=off_meta, off_v=off_v, used=used,
                stride=_round_up(used, 256), n_up_frag=n_up_frag)


def pnmix_slot_channels(hi_mask_channels: np.ndarray):
    """Slot order of the LSB plane: high channels ascending, then low ones."""
    hi = [d for d in range(D) if hi_mask_channels[d]]
    lo = [d for d in range(D) if not hi_mask_channels[d]]
    return np.array(hi + lo, dtype=np.int64), len(hi)


def pack_pnmix_page(hi_channels, codes, scale, offset, v):
    """codes [128 ch][128 t] (3-bit for high channels, 1-bit for low),
    scale/offset [128 ch] f16 bits, hi_channels bool [128]."""
    order, n_hi = pnmix_slot_channels(hi_channels)
    g = pnmix_geometry(n_hi)
    page = np.zeros(g["stride"], np.uint8)
    lsb = (codes[order] & 1).astype(np.uint8)
    page[0: 2048] = pack1_region(lsb)
    up = (codes[order[:n_hi]] >> 1).astype(np.uint8)
    reg = pack2_region(up)
    page[g["off_up"]: g["off_up"] + reg.size] = reg
    for f in range(16):
        base = g["off_meta"] + 32 * f
        page[base: base + 16] = _u16_bytes(scale[order[8 * f: 8 * f + 8]])
        page[base + 16: base + 32] = _u16_bytes(offset[order[8 * f: 8 * f + 8]])
    page[g["off_v"]: g["off_v"] + V_CODE_BYTES + V_META_BYTES] = pack_v(*v)
    return page


def unpack_pnmix_page(page, hi_channels):
    order, n_hi = pnmix_slot_channels(hi_channels)
    g = pnmix_geometry(n_hi)
    page = np.asarray(page, np.uint8)
    lsb = unpack1_region(page[0: 2048], D)
    up = unpack2_region(page[g["off_up"]: g["off_up"] + 256 * g["n_up_frag"]], n_hi)
    codes = np.zeros((D, PAGE), np.uint8)
    codes[order] = lsb
    codes[order[:n_hi]] |= (up << 1).astype(np.uint8)
    scale = np.zeros(D, np.uint16)
    offset = np.zeros(D, np.uint16)
    for f in range(16):
        base = g["off_meta"] + 32 * f
        scale[order[8 * f: 8 * f + 8]] = _bytes_u16(page[base: base + 16])
        offset[order[8 * f: 8 * f + 8]] = _bytes_u16(page[base + 16: base + 32])
    v = unpack_v(page[g["off_v"]:])
    return dict(codes=codes, scale=scale, offset=offset, v=v)


# --------------------------------------------------------------- QJL
def qjl_geometry(m: int, m_out: int = 0):
    """QJL page: sign bits of m (+ m_out outlier-instance) rows, 16 B per row
    (fragment order of pack1_region), the binary16 norms, with the outlier
    split a second norm array, then the value region."""
    off_norm = 16 * (m + m_out)
    off_norm_o = off_norm + 256
    off_v = off_norm + (512 if m_out else 256)
    used = off_v + V_CODE_BYTES + V_META_BYTES
    return dict(off_norm=off_norm, off_norm_o=off_norm_o, off_v=off_v, used=used, stride=_round_up(used, 256))


def norm_position(t: int) -> int:
    """Index (in f16 units) of token t's norm: tokens 16i + 4a + e at 32a + 4i + e."""
    i, rem = divmod(t, 16)
    a, e = divmod(rem, 4)
    return 32 * a + 4 * i + e


def _put_norms(page, off, norms):
    nv = np.zeros(PAGE, np.uint16)
    for t in range(PAGE):
        nv[norm_position(t)] = norms[t]
    page[off: off + 256] = _u16_bytes(nv)


def _get_norms(page, off):
    nv = _bytes_u16(page[off: off + 256])
    return np.array([nv[norm_position(t)] for t in range(PAGE)], dtype=np.uint16)


def pack_qjl_page(m, bits, norms, v, norms_out=None):
    """bits [m (+ m_out)][128 t] sign bits (1 = non-negative); norms [128] f16
    bits; norms_out: the outlier instance's norms (with m_out rows of bits)."""
    bits = np.asarray(bits, np.uint8)
    m_out = bits.shape[0] - m
    g = qjl_geometry(m, m_out)
    page = np.zeros(g["stride"], np.uint8)
    page[0: 16 * (m + m_out)] = pack1_region(bits)
    _put_norms(page, g["off_norm"], norms)
    if m_out:
        _put_norms(page, g["off_norm_o"], norms_out)
    page[g["off_v"]: g["off_v"] + V_CODE_BYTES + V_META_BYTES] = pack_v(*v)
    return page


def unpack_qjl_page(page, m, m_out=0):
    g = qjl_geometry(m, m_out)
    page = np.asarray(page, np.uint8)
    bits = unpack1_region(page[0: 16 * (m + m_out)], m + m_out)
    out = dict(bits=bits, norms=_get_norms(page, g["off_norm"]), v=unpack_v(page[g["off_v"]:]))
    if m_out:
        out["norms_out"] = _get_norms(page, g["off_norm_o"])
    return out
