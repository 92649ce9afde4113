"""ctypes wrapper around the fp64 CPU oracle (oracle.c).

TEST INFRASTRUCTURE: only tests/, the package smoke check and the bench's
CPU-baseline leg import this module.  The HIP product path never does.

Every function takes numpy arrays (inputs exactly as the decode step receives
them) and returns float64 results.  The arithmetic lives in oracle.c.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "liboracle.so")
_lib = None

Q8_0, Q4_K, Q5_K, Q6_K = 8, 12, 13, 14
KV_F32, KV_F16, KV_Q8_0 = 0, 1, 2


def lib() -> C.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            from . import build as _b
            _b.build()
        _lib = C.CDLL(_SO)
        _declare(_lib)
    return _lib


_p = C.c_void_p
_i = C.c_int
_i64 = C.c_int64
_d = C.c_double


class LayerCfg(C.Structure):
    _fields_ = [("hidden", _i), ("n_q_heads", _i), ("n_kv_heads", _i), ("head_dim", _i), ("ffn", _i),
                ("rms_eps", _d), ("rope_theta", _d), ("rope_style", _i), ("qk_norm", _i), ("kv_dtype", _i)]


class LayerW(C.Structure):
    _fields_ = [("attn_norm", _p), ("ffn_norm", _p), ("q_norm", _p), ("k_norm", _p),
                ("wq", _p), ("wk", _p), ("wv", _p), ("wo", _p), ("w_gate", _p), ("w_up", _p), ("w_down", _p),
                ("tq", _i), ("tk", _i), ("tv", _i), ("to", _i), ("tgate", _i), ("tup", _i), ("tdown", _i)]


class LayerTaps(C.Structure):
    _fields_ = [("q", _p), ("k", _p), ("v", _p), ("attn", _p), ("h1", _p), ("act", _p)]


def _declare(L: C.CDLL) -> None:
    L.orc_f16_to_f64.argtypes = [C.c_uint16]
    L.orc_f16_to_f64.restype = _d
    L.orc_f64_to_f16.argtypes = [_d]
    L.orc_f64_to_f16.restype = C.c_uint16
    for n in ("orc_q4k_dequant", "orc_q6k_dequant", "orc_q8_0_dequant", "orc_q5k_dequant"):
        getattr(L, n).argtypes = [_p, _i64, _p]
        getattr(L, n).restype = None
    L.orc_num_threads.argtypes = []
    L.orc_num_threads.restype = _i
    L.orc_gemm.argtypes = [_i, _p, _p, _p, _i, _i, _i]
    L.orc_gemm.restype = _i
    L.orc_rmsnorm.argtypes = [_p, _p, _d, _i, _p]
    L.orc_rmsnorm.restype = None
    L.orc_rope.argtypes = [_p, _i, _i, _d, _i]
    L.orc_rope.restype = None
    L.orc_silu.argtypes = [_d]
    L.orc_silu.restype = _d
    L.orc_head_bytes.argtypes = [_i, _i]
    L.orc_head_bytes.restype = _i64
    L.orc_q8_0_quantize_block.argtypes = [_p, _p, _p]
    L.orc_q8_0_quantize_block.restype = None
    L.orc_kv_append.argtypes = [_p, _i, _i, _i, _i, _p, _i, _p]
    L.orc_kv_append.restype = None
    L.orc_gather_kv.argtypes = [_p, _i, _i, _i, _i, _p, _i, _p, _i, _p]
    L.orc_gather_kv.restype = None
    L.orc_attend_head.argtypes = [_p, _p, _p, _i, _i, _i, _i, _p]
    L.orc_attend_head.restype = None
    L.orc_attend_partial.argtypes = [_p, _p, _p, _i, _i, _i, _i, _i, _p, _p, _p]
    L.orc_attend_partial.restype = None
    L.orc_lse_merge.argtypes = [_p, _p, _p, _i, _i, _p]
    L.orc_lse_merge.restype = None
    L.orc_paged_attention.argtypes = [_p, _p, _p, _i, _p, _i, _p, _i, _i, _i, _i, _p]
    L.orc_paged_attention.restype = None
    L.orc_decode_layer.argtypes = [C.POINTER(LayerCfg), C.POINTER(LayerW), _p, _p, _p, _p, _i, _p, _i,
                                   C.POINTER(LayerTaps)]
    L.orc_decode_layer.restype = _i
    L.orc_output_head.argtypes = [_p, _p, _d, _p, _i, _p, _i, _i, _i]
    L.orc_output_head.restype = _i
    L.orc_exp_neg.argtypes = [_d]
    L.orc_exp_neg.restype = _d
    L.orc_sample_weight.argtypes = [_d]
    L.orc_sample_weight.restype = C.c_uint32
    L.orc_sample.argtypes = [_p, _i, _i, _p, _p, _p, _p, _p, _p, _p]
    L.orc_sample.restype = _i


def num_threads() -> int:
    """OpenMP threads the oracle's parallel loops run on."""
    return int(lib().orc_num_threads())


def _ptr(a: Optional[np.ndarray]) -> Optional[int]:
    return None if a is None else a.ctypes.data


def _c(a: np.ndarray, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


# ------------------------------------------------------------------------------------ scalars

def f16_to_f64(bits: int) -> float:
    return lib().orc_f16_to_f64(int(bits) & 0xFFFF)


def f64_to_f16(x: float) -> int:
    return int(lib().orc_f64_to_f16(float(x)))


def silu(z: float) -> float:
    return lib().orc_silu(float(z))


# ------------------------------------------------------------------------------------ decoders

def dequant(kind: str, blocks: np.ndarray) -> np.ndarray:
    """kind in {"q4k", "q5k", "q6k", "q8_0"}; blocks: raw bytes (any shape) -> flat float64 values."""
    b = _c(blocks, np.uint8).reshape(-1)
    size, per = {"q4k": (144, 256), "q5k": (176, 256), "q6k": (210, 256), "q8_0": (34, 32)}[kind]
    assert b.size % size == 0
    n = b.size // size
    out = np.empty(n * per, dtype=np.float64)
    getattr(lib(), f"orc_{kind}_dequant")(_ptr(b), n, _ptr(out))
    return out


def gemm(wtype: int, w: np.ndarray, x: np.ndarray, n: int, k: int) -> np.ndarray:
    """y [B, n] = x [B, k] @ W^T with W decoded exactly (float64)."""
    x64 = _c(np.atleast_2d(x), np.float64)
    bsz = x64.shape[0]
    y = np.empty((bsz, n), dtype=np.float64)
    rc = lib().orc_gemm(wtype, _ptr(_c(w, np.uint8)), _ptr(x64), _ptr(y), bsz, n, k)
    if rc:
        raise ValueError("oracle gemm rejected its arguments")
    return y


def rmsnorm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    x64 = _c(x, np.float64).reshape(-1)
    out = np.empty_like(x64)
    lib().orc_rmsnorm(_ptr(x64), _ptr(_c(g, np.float32)), float(eps), x64.size, _ptr(out))
    return out


def rope(v: np.ndarray, pos: int, theta: float, style: int) -> np.ndarray:
    out = _c(v, np.float64).reshape(-1).copy()
    lib().orc_rope(_ptr(out), out.size, int(pos), float(theta), int(style))
    return out


def head_bytes(kv_dtype: int, d: int) -> int:
    return int(lib().orc_head_bytes(kv_dtype, d))


def q8_0_quantize_block(x: np.ndarray):
    """32 float32 values -> (int8 codes, fp16 scale bits) with the fp32 quantizer."""
    xf = _c(x, np.float32).reshape(32)
    q = np.empty(32, dtype=np.int8)
    d = np.empty(1, dtype=np.uint16)
    lib().orc_q8_0_quantize_block(_ptr(xf), _ptr(q), _ptr(d))
    return q, int(d[0])


def kv_append(pool: np.ndarray, kv_dtype: int, is_v: bool, hkv: int, d: int, bt_row: np.ndarray, pos: int,
              vec: np.ndarray) -> None:
    assert pool.flags.c_contiguous and pool.dtype == np.uint8
    lib().orc_kv_append(_ptr(pool), kv_dtype, int(is_v), hkv, d, _ptr(_c(bt_row, np.int32)), int(pos),
                        _ptr(_c(vec, np.float64)))


def gather_kv(pool: np.ndarray, kv_dtype: int, is_v: bool, hkv: int, d: int, block_table: np.ndarray,
              ctx: np.ndarray) -> np.ndarray:
    """Rows concatenated: [sum(ctx), hkv, d] float64 exact values."""
    bt = _c(block_table, np.int32)
    cl = _c(ctx, np.int32)
    out = np.empty((int(cl.sum()), hkv, d), dtype=np.float64)
    lib().orc_gather_kv(_ptr(_c(pool, np.uint8)), kv_dtype, int(is_v), hkv, d, _ptr(bt), bt.shape[1], _ptr(cl),
                        cl.size, _ptr(out))
    return out


def attend_head(q: np.ndarray, K: np.ndarray, V: np.ndarray, g: int) -> np.ndarray:
    """q [D]; K, V [n, hkv, D] contiguous -> o [D]."""
    K64, V64 = _c(K, np.float64), _c(V, np.float64)
    n, hkv, d = K64.shape
    o = np.empty(d, dtype=np.float64)
    lib().orc_attend_head(_ptr(_c(q, np.float64)), _ptr(K64), _ptr(V64), n, hkv, d, g, _ptr(o))
    return o


def attend_partial(q, K, V, t0: int, t1: int, g: int):
    K64, V64 = _c(K, np.float64), _c(V, np.float64)
    _, hkv, d = K64.shape
    o = np.empty(d, dtype=np.float64)
    m = np.empty(1)
    l_ = np.empty(1)
    lib().orc_attend_partial(_ptr(_c(q, np.float64)), _ptr(K64), _ptr(V64), t0, t1, hkv, d, g, _ptr(o), _ptr(m),
                             _ptr(l_))
    return o, float(m[0]), float(l_[0])


def lse_merge(o_s: np.ndarray, m_s: np.ndarray, l_s: np.ndarray) -> np.ndarray:
    o_s = _c(o_s, np.float64)
    s, d = o_s.shape
    o = np.empty(d, dtype=np.float64)
    lib().orc_lse_merge(_ptr(o_s), _ptr(_c(m_s, np.float64)), _ptr(_c(l_s, np.float64)), s, d, _ptr(o))
    return o


def paged_attention(q: np.ndarray, k_pool: np.ndarray, v_pool: np.ndarray, kv_dtype: int, block_table: np.ndarray,
                    ctx: np.ndarray, hkv: int) -> np.ndarray:
    """q [B, Hq, D] -> out [B, Hq, D]; row b attends its ctx[b] cached tokens."""
    q64 = _c(q, np.float64)
    bsz, hq, d = q64.shape
    bt = _c(block_table, np.int32)
    out = np.empty_like(q64)
    lib().orc_paged_attention(_ptr(q64), _ptr(_c(k_pool, np.uint8)), _ptr(_c(v_pool, np.uint8)), kv_dtype, _ptr(bt),
                              bt.shape[1], _ptr(_c(ctx, np.int32)), bsz, hq, hkv, d, _ptr(out))
    return out


# ------------------------------------------------------------------------------------ layer / stack

def _cfg(w) -> LayerCfg:
    return LayerCfg(w.hidden, w.n_q_heads, w.n_kv_heads, w.head_dim, w.ffn, float(w.rms_eps), float(w.rope_theta),
                    int(w.rope_style), int(bool(w.qk_norm)), int(w.kv_dtype))


def decode_layer(workload, lw, k_pool: np.ndarray, v_pool: np.ndarray, x: np.ndarray, block_table: np.ndarray,
                 ctx: np.ndarray, taps: bool = False):
    """One decode layer.  k_pool / v_pool (uint8, C-contiguous) receive the appended
    token in place.  x: [B, H] (any float dtype) -> new x [B, H] float64.  With
    taps=True also returns a dict of intermediates."""
    keep = []

    def arr(a, dt):
        if a is None:
            return None
        c = _c(a, dt)
        keep.append(c)
        return _ptr(c)

    W = LayerW(arr(lw.attn_norm, np.float32), arr(lw.ffn_norm, np.float32), arr(lw.q_norm, np.float32),
               arr(lw.k_norm, np.float32), arr(lw.wq, np.uint8), arr(lw.wk, np.uint8), arr(lw.wv, np.uint8),
               arr(lw.wo, np.uint8), arr(lw.w_gate, np.uint8), arr(lw.w_up, np.uint8), arr(lw.w_down, np.uint8),
               lw.tq, lw.tk, lw.tv, lw.to, lw.tgate, lw.tup, lw.tdown)
    x64 = _c(x, np.float64).copy()
    bsz = x64.shape[0]
    assert k_pool.flags.c_contiguous and v_pool.flags.c_contiguous
    bt = _c(block_table, np.int32)
    t = None
    tp = None
    if taps:
        qd, kvd = workload.n_q_heads * workload.head_dim, workload.n_kv_heads * workload.head_dim
        t = dict(q=np.empty((bsz, qd)), k=np.empty((bsz, kvd)), v=np.empty((bsz, kvd)), attn=np.empty((bsz, qd)),
                 h1=np.empty((bsz, workload.hidden)), act=np.empty((bsz, workload.ffn)))
        tp = C.pointer(LayerTaps(*[_ptr(t[k]) for k in ("q", "k", "v", "attn", "h1", "act")]))
    rc = lib().orc_decode_layer(C.byref(_cfg(workload)), C.byref(W), _ptr(k_pool), _ptr(v_pool), _ptr(x64),
                                _ptr(bt), bt.shape[1], _ptr(_c(ctx, np.int32)), bsz, tp)
    if rc:
        raise ValueError("oracle decode_layer rejected its arguments")
    return (x64, t) if taps else x64


def output_head(x: np.ndarray, norm: np.ndarray, eps: float, w: np.ndarray, wtype: int, vocab: int) -> np.ndarray:
    x64 = _c(np.atleast_2d(x), np.float64)
    bsz, h = x64.shape
    out = np.empty((bsz, vocab), dtype=np.float64)
    rc = lib().orc_output_head(_ptr(x64), _ptr(_c(norm, np.float32)), float(eps), _ptr(_c(w, np.uint8)), wtype,
                               _ptr(out), bsz, h, vocab)
    if rc:
        raise ValueError("oracle output_head rejected its arguments")
    return out


def exp_neg(d: float) -> float:
    """e^d for -22 <= d <= 0 as the sampler evaluates it (fp64)."""
    return float(lib().orc_exp_neg(float(d)))


def sample_weight(d: float) -> int:
    """Fixed-point weight floor(2^31 e^d) of a scaled logit difference d (0 below -22 or for NaN)."""
    return int(lib().orc_sample_weight(float(d)))


def sample(logits: np.ndarray, temperature, top_p, top_k, u, diag: bool = False):
    """One token per row of float32 logits [B, vocab]; per-row temperature, top_p, top_k, uniform u.

    With diag=True also returns (Wk, Wp): the kept weight after the top-k and the top-p cuts."""
    lg = _c(np.atleast_2d(logits), np.float32)
    bsz, vocab = lg.shape
    t = _c(np.broadcast_to(np.asarray(temperature, dtype=np.float64), (bsz,)), np.float64)
    p = _c(np.broadcast_to(np.asarray(top_p, dtype=np.float64), (bsz,)), np.float64)
    k = _c(np.broadcast_to(np.asarray(top_k, dtype=np.int32), (bsz,)), np.int32)
    uu = _c(np.broadcast_to(np.asarray(u, dtype=np.float64), (bsz,)), np.float64)
    tok = np.empty(bsz, dtype=np.int32)
    wk = np.empty(bsz, dtype=np.uint64)
    wp = np.empty(bsz, dtype=np.uint64)
    rc = lib().orc_sample(_ptr(lg), bsz, vocab, _ptr(t), _ptr(p), _ptr(k), _ptr(uu), _ptr(tok), _ptr(wk), _ptr(wp))
    if rc:
        raise ValueError("oracle sample rejected its arguments")
    return (tok, wk, wp) if diag else tok


def decode_stack(workload, layers: Sequence, k_pools: Sequence[np.ndarray], v_pools: Sequence[np.ndarray],
                 x: np.ndarray, block_table: np.ndarray, ctx: np.ndarray, head=None):
    """All layers in order (pools modified in place); returns (per-layer outputs, logits or None)."""
    outs = []
    cur = x
    for lw, kp, vp in zip(layers, k_pools, v_pools):
        cur = decode_layer(workload, lw, kp, vp, cur, block_table, ctx)
        outs.append(cur)
    logits = None
    if head is not None:
        norm, w = head
        logits = output_head(cur, norm, workload.rms_eps, w, workload.w_head, workload.vocab)
    return outs, logits


def verify_stack(workload, layers: Sequence, k_pools: Sequence[np.ndarray], v_pools: Sequence[np.ndarray],
                 x: np.ndarray, block_table: np.ndarray, ctx: np.ndarray, t: int, head=None):
    """T tokens per sequence in one step (speculative verification; Leone, "What ships").

    x holds B*T rows, token j of sequence b in row b*T + j at position ctx[b] + j.  Layer by
    layer, the tokens go through decode_layer in token order, so token j's attention sees the
    K/V that tokens 0..j-1 of the same step appended: the step equals T decode steps.  Pools
    are modified in place.  Returns (per-layer outputs [B*T, H], logits or None)."""
    ctx = np.asarray(ctx, dtype=np.int32)
    bsz = len(ctx)
    h = workload.hidden
    cur = np.asarray(x, dtype=np.float64).reshape(bsz, t, h)
    outs = []
    for lw, kp, vp in zip(layers, k_pools, v_pools):
        nxt = np.empty_like(cur)
        for j in range(t):
            nxt[:, j] = decode_layer(workload, lw, kp, vp, cur[:, j], block_table, ctx + j)
        cur = nxt
        outs.append(cur.reshape(bsz * t, h).copy())
    logits = None
    if head is not None:
        norm, w = head
        logits = output_head(cur.reshape(bsz * t, h), norm, workload.rms_eps, w, workload.w_head, workload.vocab)
    return outs, logits


def spec_accept(sampled: np.ndarray, draft: np.ndarray) -> np.ndarray:
    """Accepted proposals per sequence: the leading positions j < T-1 where the target's token
    after position j equals the step's input token j+1 (the proposal there)."""
    sampled = np.atleast_2d(sampled)
    draft = np.atleast_2d(draft)
    out = np.zeros(sampled.shape[0], dtype=np.int32)
    for b in range(sampled.shape[0]):
        n = 0
        while n < sampled.shape[1] - 1 and sampled[b, n] == draft[b, n + 1]:
            n += 1
        out[b] = n
    return out


def mixed_stack(workload, layers: Sequence, k_pools: Sequence[np.ndarray], v_pools: Sequence[np.ndarray],
                x: np.ndarray, block_table: np.ndarray, row_seq: np.ndarray, row_pos: np.ndarray, head=None):
    """A step of rows placed by (sequence, position) (Leone, "What ships": chunked prefill and
    continuous decode batching): decode rows, verification runs and prompt chunks together.

    Layer by layer, the rows go through decode_layer one at a time in increasing position, each
    with its own sequence's block table row, so a sequence's earlier tokens are appended before
    its later ones attend.  Pools are modified in place.  Returns (per-layer outputs [rows, H],
    logits or None)."""
    row_seq = np.asarray(row_seq, dtype=np.int64)
    row_pos = np.asarray(row_pos, dtype=np.int32)
    order = np.argsort(row_pos, kind="stable")
    cur = np.asarray(x, dtype=np.float64).copy()
    outs = []
    for lw, kp, vp in zip(layers, k_pools, v_pools):
        nxt = np.empty_like(cur)
        for r in order:
            s = int(row_seq[r])
            nxt[r] = decode_layer(workload, lw, kp, vp, cur[r:r + 1], block_table[s:s + 1], row_pos[r:r + 1])[0]
        cur = nxt
        outs.append(cur.copy())
    logits = None
    if head is not None:
        norm, w = head
        logits = output_head(cur, norm, workload.rms_eps, w, workload.w_head, workload.vocab)
    return outs, logits
