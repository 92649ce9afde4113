"""Second, independent CPU implementation used to pin the oracle.

Written in numpy from the same definitions as oracle.c but sharing no code with
it: block packers/unpackers for the public GGUF Q4_K / Q6_K / q8_0 layouts, and a
brute-force decode layer for small shapes.  Used only by the tests.
"""
from __future__ import annotations

import math

import numpy as np

PAGE = 16


# ----------------------------------------------------------------------------- packers

def pack_q4k_scales(sc, mn) -> bytes:
    """Eight 6-bit scales and eight 6-bit mins -> the 12 packed bytes.

    Bytes 0-3 hold sc[0..3] in their low 6 bits and the top 2 bits of sc[4..7];
    bytes 4-7 hold m[0..3] and the top 2 bits of m[4..7]; bytes 8-11 hold the low
    4 bits of sc[4..7] (low nibble) and of m[4..7] (high nibble)."""
    s = [0] * 12
    for j in range(4):
        s[j] = (sc[j] & 63) | ((sc[j + 4] >> 4) << 6)
        s[j + 4] = (mn[j] & 63) | ((mn[j + 4] >> 4) << 6)
        s[j + 8] = (sc[j + 4] & 15) | ((mn[j + 4] & 15) << 4)
    return bytes(s)


def unpack_q4k_scales(s: bytes):
    sc = [0] * 8
    mn = [0] * 8
    for j in range(4):
        sc[j] = s[j] & 63
        mn[j] = s[j + 4] & 63
        sc[j + 4] = (s[j + 8] & 15) | ((s[j] >> 6) << 4)
        mn[j + 4] = (s[j + 8] >> 4) | ((s[j + 4] >> 6) << 4)
    return sc, mn


def f16_bits(x: float) -> int:
    return int(np.array([x], dtype=np.float16).view(np.uint16)[0])


def pack_q4k_block(d: float, dmin: float, sc, mn, q) -> bytes:
    """q: 256 ints in [0,16) in logical weight order."""
    qs = [0] * 128
    for c in range(4):
        for l in range(32):
            qs[32 * c + l] = (q[64 * c + l] & 15) | ((q[64 * c + 32 + l] & 15) << 4)
    return (f16_bits(d).to_bytes(2, "little") + f16_bits(dmin).to_bytes(2, "little") + pack_q4k_scales(sc, mn)
            + bytes(qs))


def pack_q6k_block(d: float, scales, q) -> bytes:
    """scales: 16 ints in [-128,128); q: 256 ints in [0,64) in logical weight order."""
    ql = [0] * 128
    qh = [0] * 64
    for h in range(2):
        for l in range(32):
            q0, q1, q2, q3 = (q[128 * h + l + 32 * r] for r in range(4))
            ql[64 * h + l] = (q0 & 15) | ((q2 & 15) << 4)
            ql[64 * h + 32 + l] = (q1 & 15) | ((q3 & 15) << 4)
            qh[32 * h + l] = (q0 >> 4) | ((q1 >> 4) << 2) | ((q2 >> 4) << 4) | ((q3 >> 4) << 6)
    return bytes(ql) + bytes(qh) + bytes((s & 255) for s in scales) + f16_bits(d).to_bytes(2, "little")


def pack_q5k_block(d: float, dmin: float, sc, mn, q) -> bytes:
    """q: 256 ints in [0,32) in logical weight order (the Q4_K nibble order, fifth bits apart)."""
    qs = [0] * 128
    qh = [0] * 32
    for c in range(4):
        for l in range(32):
            a, b = q[64 * c + l], q[64 * c + 32 + l]
            qs[32 * c + l] = (a & 15) | ((b & 15) << 4)
            qh[l] |= ((a >> 4) & 1) << (2 * c) | ((b >> 4) & 1) << (2 * c + 1)
    return (f16_bits(d).to_bytes(2, "little") + f16_bits(dmin).to_bytes(2, "little") + pack_q4k_scales(sc, mn)
            + bytes(qh) + bytes(qs))


def pack_q8_0_block(d: float, q) -> bytes:
    return f16_bits(d).to_bytes(2, "little") + bytes((v & 255) for v in q)


# ----------------------------------------------------------------------------- vectorized decoders

def _f16(u16: np.ndarray) -> np.ndarray:
    return u16.astype(np.uint16).view(np.float16).astype(np.float64)


def decode_q4k(blocks: np.ndarray) -> np.ndarray:
    """[n, 144] uint8 -> [n, 256] float64 (exact)."""
    b = blocks.reshape(-1, 144)
    d = _f16(b[:, 0].astype(np.uint16) | (b[:, 1].astype(np.uint16) << 8))
    dmin = _f16(b[:, 2].astype(np.uint16) | (b[:, 3].astype(np.uint16) << 8))
    s = b[:, 4:16].astype(np.int64)
    sc = np.empty((b.shape[0], 8), np.int64)
    mn = np.empty((b.shape[0], 8), np.int64)
    sc[:, :4] = s[:, 0:4] & 63
    mn[:, :4] = s[:, 4:8] & 63
    sc[:, 4:] = (s[:, 8:12] & 15) | ((s[:, 0:4] >> 6) << 4)
    mn[:, 4:] = (s[:, 8:12] >> 4) | ((s[:, 4:8] >> 6) << 4)
    qs = b[:, 16:144].astype(np.int64).reshape(-1, 4, 32)
    q = np.empty((b.shape[0], 4, 2, 32), np.int64)
    q[:, :, 0, :] = qs & 15
    q[:, :, 1, :] = qs >> 4
    q = q.reshape(-1, 8, 32)  # sub-block j = 2c + (high nibble)
    w = d[:, None, None] * sc[:, :, None] * q - dmin[:, None, None] * mn[:, :, None]
    return w.reshape(-1, 256)


def decode_q5k(blocks: np.ndarray) -> np.ndarray:
    """[n, 176] uint8 -> [n, 256] float64 (exact)."""
    b = blocks.reshape(-1, 176)
    d = _f16(b[:, 0].astype(np.uint16) | (b[:, 1].astype(np.uint16) << 8))
    dmin = _f16(b[:, 2].astype(np.uint16) | (b[:, 3].astype(np.uint16) << 8))
    sc, mn = np.empty((b.shape[0], 8), np.int64), np.empty((b.shape[0], 8), np.int64)
    for r in range(b.shape[0]):
        sc[r], mn[r] = unpack_q4k_scales(bytes(b[r, 4:16]))
    qh = b[:, 16:48].astype(np.int64)  # [n, l]
    qs = b[:, 48:176].astype(np.int64).reshape(-1, 4, 32)
    q = np.empty((b.shape[0], 4, 2, 32), np.int64)
    for c in range(4):
        q[:, c, 0] = (qs[:, c] & 15) + 16 * ((qh >> (2 * c)) & 1)
        q[:, c, 1] = (qs[:, c] >> 4) + 16 * ((qh >> (2 * c + 1)) & 1)
    q = q.reshape(-1, 8, 32)
    w = d[:, None, None] * sc[:, :, None] * q - dmin[:, None, None] * mn[:, :, None]
    return w.reshape(-1, 256)


def decode_q6k(blocks: np.ndarray) -> np.ndarray:
    b = blocks.reshape(-1, 210)
    ql = b[:, 0:128].astype(np.int64).reshape(-1, 2, 2, 32)  # [n, half, lo/hi 32, l]
    qh = b[:, 128:192].astype(np.int64).reshape(-1, 2, 32)
    sc = b[:, 192:208].view(np.int8).astype(np.int64)
    d = _f16(b[:, 208].astype(np.uint16) | (b[:, 209].astype(np.uint16) << 8))
    q = np.empty((b.shape[0], 2, 4, 32), np.int64)
    q[:, :, 0] = (ql[:, :, 0] & 15) | (((qh >> 0) & 3) << 4)
    q[:, :, 1] = (ql[:, :, 1] & 15) | (((qh >> 2) & 3) << 4)
    q[:, :, 2] = (ql[:, :, 0] >> 4) | (((qh >> 4) & 3) << 4)
    q[:, :, 3] = (ql[:, :, 1] >> 4) | (((qh >> 6) & 3) << 4)
    q = q.reshape(-1, 256)
    return d[:, None] * np.repeat(sc, 16, axis=1) * (q - 32)


def decode_q8_0(blocks: np.ndarray) -> np.ndarray:
    b = blocks.reshape(-1, 34)
    d = _f16(b[:, 0].astype(np.uint16) | (b[:, 1].astype(np.uint16) << 8))
    return d[:, None] * b[:, 2:].view(np.int8).astype(np.float64)


def decode_matrix(wtype: int, w: np.ndarray, n: int, k: int) -> np.ndarray:
    if wtype == 12:
        return decode_q4k(w.reshape(n * (k // 256), 144)).reshape(n, k)
    if wtype == 14:
        return decode_q6k(w.reshape(n * (k // 256), 210)).reshape(n, k)
    if wtype == 13:
        return decode_q5k(w.reshape(n * (k // 256), 176)).reshape(n, k)
    if wtype == 8:
        return decode_q8_0(w.reshape(n * (k // 32), 34)).reshape(n, k)
    raise ValueError(wtype)


# ----------------------------------------------------------------------------- paged KV

def head_bytes(kv_dtype: int, d: int) -> int:
    return {0: PAGE * d * 4, 1: PAGE * d * 2, 2: PAGE * d + PAGE * (d // 32) * 2}[kv_dtype]


def decode_page_head(raw: np.ndarray, kv_dtype: int, is_v: bool, d: int) -> np.ndarray:
    """One (page, head) byte block -> [16 tokens, d] float64."""
    if kv_dtype == 0:
        e = raw.view(np.float32).astype(np.float64)
    elif kv_dtype == 1:
        e = raw.view(np.float16).astype(np.float64)
    else:
        codes = raw[:PAGE * d].view(np.int8).astype(np.float64)
        sc = raw[PAGE * d:].view(np.float16).astype(np.float64).reshape(PAGE, d // 32)
        e = codes
    e = e.reshape(d, PAGE).T if is_v else e.reshape(PAGE, d)
    if kv_dtype == 2:
        e = e * np.repeat(sc, 32, axis=1)
    return e


def gather_row(pool: np.ndarray, kv_dtype: int, is_v: bool, hkv: int, d: int, bt_row, n_tok: int) -> np.ndarray:
    hb = head_bytes(kv_dtype, d)
    out = np.empty((n_tok, hkv, d))
    for j in range((n_tok + PAGE - 1) // PAGE):
        page = pool[int(bt_row[j])]
        for g in range(hkv):
            e = decode_page_head(page[g * hb:(g + 1) * hb], kv_dtype, is_v, d)
            n = min(PAGE, n_tok - j * PAGE)
            out[j * PAGE:j * PAGE + n, g] = e[:n]
    return out


# ----------------------------------------------------------------------------- brute force layer

def rms(x, g, eps):
    return x / np.sqrt(np.mean(x * x) + eps) * g.astype(np.float64)


def rope(v, p, theta, neox: bool):
    d = v.shape[-1]
    out = v.copy()
    i = np.arange(d // 2)
    ang = p * theta ** (-2.0 * i / d)
    c, s = np.cos(ang), np.sin(ang)
    if neox:
        a, b = v[..., :d // 2], v[..., d // 2:]
        out[..., :d // 2] = a * c - b * s
        out[..., d // 2:] = a * s + b * c
    else:
        a, b = v[..., 0::2], v[..., 1::2]
        out[..., 0::2] = a * c - b * s
        out[..., 1::2] = a * s + b * c
    return out


def store_round(v: np.ndarray, kv_dtype: int) -> np.ndarray:
    """Value the cache holds after storing v (q8_0: per 32-block, quantized in fp32)."""
    if kv_dtype == 0:
        return v.astype(np.float32).astype(np.float64)
    if kv_dtype == 1:
        return v.astype(np.float16).astype(np.float64)
    out = np.empty_like(v)
    flat = v.reshape(-1, 32).astype(np.float32)
    o = out.reshape(-1, 32)
    for i, blk in enumerate(flat):
        amax = np.float32(np.max(np.abs(blk)))
        dd = np.float32(amax / np.float32(127.0))
        if dd == 0:
            o[i] = 0.0
            continue
        r = blk / dd
        q = np.clip(np.sign(r) * np.floor(np.abs(r) + np.float32(0.5)), -127, 127)
        o[i] = q.astype(np.float64) * float(np.float16(dd))
    return out


def silu(z):
    return z / (1.0 + np.exp(-z))


def brute_layer(wl, lw, k_pool, v_pool, x, bt, ctx):
    """Numpy brute force of one decode layer (pools are read, not modified)."""
    H, hq, hkv, d, F = wl.hidden, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.ffn
    Wq = decode_matrix(lw.tq, lw.wq, hq * d, H)
    Wk = decode_matrix(lw.tk, lw.wk, hkv * d, H)
    Wv = decode_matrix(lw.tv, lw.wv, hkv * d, H)
    Wo = decode_matrix(lw.to, lw.wo, H, hq * d)
    Wg = decode_matrix(lw.tgate, lw.w_gate, F, H)
    Wu = decode_matrix(lw.tup, lw.w_up, F, H)
    Wd = decode_matrix(lw.tdown, lw.w_down, H, F)
    out = np.empty((x.shape[0], H))
    for b in range(x.shape[0]):
        xb = x[b].astype(np.float64)
        p = int(ctx[b])
        xn = rms(xb, lw.attn_norm, wl.rms_eps)
        q = (Wq @ xn).reshape(hq, d)
        k = (Wk @ xn).reshape(hkv, d)
        v = (Wv @ xn).reshape(hkv, d)
        if wl.qk_norm:
            q = np.stack([rms(q[h], lw.q_norm, wl.rms_eps) for h in range(hq)])
            k = np.stack([rms(k[h], lw.k_norm, wl.rms_eps) for h in range(hkv)])
        neox = wl.rope_style == 0
        q = rope(q, p, wl.rope_theta, neox)
        k = rope(k, p, wl.rope_theta, neox)
        K = gather_row(k_pool, wl.kv_dtype, False, hkv, d, bt[b], p)
        V = gather_row(v_pool, wl.kv_dtype, True, hkv, d, bt[b], p)
        K = np.concatenate([K, store_round(k, wl.kv_dtype)[None]], axis=0)
        V = np.concatenate([V, store_round(v, wl.kv_dtype)[None]], axis=0)
        o = np.empty((hq, d))
        for h in range(hq):
            g = h // (hq // hkv)
            s = K[:, g, :] @ q[h] / math.sqrt(d)
            wts = np.exp(s - s.max())
            wts /= wts.sum()
            o[h] = wts @ V[:, g, :]
        x1 = xb + Wo @ o.reshape(-1)
        xn2 = rms(x1, lw.ffn_norm, wl.rms_eps)
        a = silu(Wg @ xn2) * (Wu @ xn2)
        out[b] = x1 + Wd @ a
    return out
