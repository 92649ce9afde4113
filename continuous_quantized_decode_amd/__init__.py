"""Python binding of libgr, the MI355X (gfx950) continuous-batched quantized decode step.

Thin ctypes marshalling over the C ABI in include/gr.h: every function below takes
torch tensors (device memory) and calls the C entry point of the same name on the
current torch stream.  All arithmetic runs in the HIP kernels of libgr.so; torch
only supplies memory and streams.  There is no CPU fallback: without the built
library, or without a gfx950 device, calls raise.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional, Sequence

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgr.so")

GR_OK = 0
W_Q8_0, W_Q4_K, W_Q5_K, W_Q6_K = 8, 12, 13, 14
KV_F32, KV_F16, KV_Q8_0 = 0, 1, 2
ROPE_NEOX, ROPE_NORM = 0, 1
PAGE_SIZE = 16

_lib = None


class GrError(RuntimeError):
    def __init__(self, fn: str, status: int):
        msg = _load().gr_status_str(status).decode()
        if status == -8:
            msg += f" (hipError {_load().gr_last_hip_error()})"
        super().__init__(f"{fn}: {msg} [{status}]")
        self.status = status


_p = C.c_void_p
_i = C.c_int
_i64 = C.c_int64
_sz = C.c_size_t


class AttnMeta(C.Structure):
    _fields_ = [("n_q_heads", _i), ("n_kv_heads", _i), ("head_dim", _i), ("page_size", _i), ("kv_dtype", _i),
                ("num_pages", _i), ("max_blocks_per_row", _i), ("max_ctx", _i), ("scale", C.c_float)]


class LayerCfg(C.Structure):
    _fields_ = [("hidden", _i), ("n_q_heads", _i), ("n_kv_heads", _i), ("head_dim", _i), ("ffn", _i),
                ("rms_eps", C.c_float), ("rope_theta", C.c_double), ("rope_style", _i), ("qk_norm", _i),
                ("kv_dtype", _i), ("page_size", _i)]


class LayerWeights(C.Structure):
    _fields_ = [("attn_norm", _p), ("ffn_norm", _p), ("q_norm", _p), ("k_norm", _p), ("wq", _p), ("wk", _p),
                ("wv", _p), ("wo", _p), ("w_gate", _p), ("w_up", _p), ("w_down", _p), ("tq", _i), ("tk", _i),
                ("tv", _i), ("to", _i), ("tgate", _i), ("tup", _i), ("tdown", _i)]


def _load() -> C.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m continuous_quantized_decode_amd.build`")
    L = C.CDLL(LIB_PATH)
    L.gr_abi_version.restype = _i
    L.gr_status_str.restype = C.c_char_p
    L.gr_status_str.argtypes = [_i]
    L.gr_last_hip_error.restype = _i
    L.gr_kv_head_bytes.restype = _i64
    L.gr_kv_head_bytes.argtypes = [_i, _i]
    for n in ("gr_q4k_dequant", "gr_q6k_dequant", "gr_q8_0_dequant"):
        getattr(L, n).argtypes = [_p, _i64, _p, _p]
        getattr(L, n).restype = _i
    L.gr_gemm_workspace_size.argtypes = [_i, _i, _i]
    L.gr_gemm_workspace_size.restype = _sz
    L.gr_gemm_launch_shape.argtypes = [_i, _i, _i, _i, _i] + [C.POINTER(_i)] * 6
    L.gr_gemm_launch_shape.restype = _i
    for n in ("gr_q4k_gemm", "gr_q6k_gemm", "gr_q5k_gemm", "gr_q8_0_gemm"):
        getattr(L, n).argtypes = [_p, _p, _p, _i, _i, _i, _p, _sz, _p]
        getattr(L, n).restype = _i
    L.gr_stream_read.argtypes = [_p, _sz, _p, _p]
    L.gr_stream_read.restype = _i
    L.gr_paged_decode_attn_workspace_size.argtypes = [C.POINTER(AttnMeta), _i]
    L.gr_paged_decode_attn_workspace_size.restype = _sz
    L.gr_paged_decode_attn.argtypes = [_p, _p, _p, _p, _p, _p, _i, C.POINTER(AttnMeta), _p, _sz, _p]
    L.gr_paged_decode_attn.restype = _i
    L.gr_paged_decode_attn_noalloc.argtypes = [_p, _p, _p, _p, _p, _p, _i, C.POINTER(AttnMeta), _p]
    L.gr_paged_decode_attn_noalloc.restype = _i
    L.gr_attn_launch_shape.argtypes = [_i, _i, _i, _i, C.POINTER(_i), C.POINTER(_i), C.POINTER(_i),
                                       C.POINTER(C.c_longlong)]
    L.gr_attn_launch_shape.restype = _i
    L.gr_paged_gather_kv.argtypes = [_p, _i, _p, _p, _i, C.POINTER(AttnMeta), _p, _p]
    L.gr_paged_gather_kv.restype = _i
    L.gr_decode_layer_workspace_size.argtypes = [C.POINTER(LayerCfg), _i, _i]
    L.gr_decode_layer_workspace_size.restype = _sz
    L.gr_decode_layer.argtypes = [C.POINTER(LayerCfg), C.POINTER(LayerWeights), _p, _p, _i, _p, _p, _i, _p, _i, _i,
                                  _p, _sz, _p]
    L.gr_decode_layer.restype = _i
    L.gr_output_head_workspace_size.argtypes = [_i, _i, _i]
    L.gr_output_head_workspace_size.restype = _sz
    L.gr_output_head.argtypes = [_p, _p, C.c_float, _p, _i, _p, _i, _i, _i, _p, _sz, _p]
    L.gr_output_head.restype = _i
    L.gr_decode_stack_workspace_size.argtypes = [C.POINTER(LayerCfg), _i, _i, _i]
    L.gr_decode_stack_workspace_size.restype = _sz
    L.gr_decode_stack.argtypes = [C.POINTER(LayerCfg), C.POINTER(LayerWeights), _i, C.POINTER(_p), C.POINTER(_p), _i,
                                  _p, _p, _i, _p, _i, _i, _p, _p, _i, _i, _p, _p, _sz, _p]
    L.gr_decode_stack.restype = _i
    L.gr_decode_stack_probed.argtypes = list(L.gr_decode_stack.argtypes) + [_i, _i, C.POINTER(_p), C.POINTER(_p)]
    L.gr_decode_stack_probed.restype = _i
    L.gr_verify_stack_workspace_size.argtypes = [C.POINTER(LayerCfg), _i, _i, _i, _i]
    L.gr_verify_stack_workspace_size.restype = _sz
    L.gr_verify_stack.argtypes = [C.POINTER(LayerCfg), C.POINTER(LayerWeights), _i, C.POINTER(_p), C.POINTER(_p), _i,
                                  _p, _p, _i, _p, _i, _i, _i, _p, _p, _i, _i, _p, _p, _sz, _p]
    L.gr_verify_stack.restype = _i
    L.gr_mixed_stack_workspace_size.argtypes = [C.POINTER(LayerCfg), _i, _i, _i]
    L.gr_mixed_stack_workspace_size.restype = _sz
    L.gr_mixed_stack.argtypes = [C.POINTER(LayerCfg), C.POINTER(LayerWeights), _i, C.POINTER(_p), C.POINTER(_p), _i,
                                 _p, _p, _i, _p, _p, _i, _i, _p, _p, _i, _i, _p, _i, _p, _p, _sz, _p]
    L.gr_mixed_stack.restype = _i
    L.gr_spec_accept.argtypes = [_p, _p, _i, _i, _p, _p]
    L.gr_spec_accept.restype = _i
    L.gr_sample_workspace_size.argtypes = [_i, _i]
    L.gr_sample_workspace_size.restype = _sz
    L.gr_sample.argtypes = [_p, _i, _i, _p, _p, _p, _p, _sz, _p]
    L.gr_sample.restype = _i
    if L.gr_abi_version() != 10:
        raise ImportError("libgr ABI version mismatch")
    _lib = L
    return L


def lib() -> C.CDLL:
    return _load()


EXPORTED = ("gr_abi_version", "gr_status_str", "gr_last_hip_error", "gr_kv_head_bytes", "gr_stream_read", "gr_q4k_dequant",
            "gr_q6k_dequant", "gr_q8_0_dequant", "gr_gemm_workspace_size", "gr_gemm_launch_shape", "gr_q4k_gemm",
            "gr_q6k_gemm", "gr_q5k_gemm", "gr_q8_0_gemm",
            "gr_paged_decode_attn_workspace_size", "gr_paged_decode_attn", "gr_paged_decode_attn_noalloc", "gr_attn_launch_shape", "gr_paged_gather_kv",
            "gr_decode_layer_workspace_size", "gr_decode_layer", "gr_output_head_workspace_size", "gr_output_head",
            "gr_decode_stack_workspace_size", "gr_decode_stack", "gr_decode_stack_probed", "gr_sample_workspace_size",
            "gr_sample", "gr_verify_stack_workspace_size", "gr_verify_stack", "gr_spec_accept",
            "gr_mixed_stack_workspace_size", "gr_mixed_stack")

# gr_stage values
STAGES = ("pack", "qkv", "attn", "attn_merge", "wo", "gate_up", "down", "head")


# --------------------------------------------------------------------------- helpers

def _torch():
    import torch
    return torch


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("expected a device tensor")
    return t.data_ptr()


def _stream() -> int:
    return _torch().cuda.current_stream().cuda_stream


def _check(fn: str, status: int) -> None:
    if status != GR_OK:
        raise GrError(fn, status)


def workspace(nbytes: int, device=None):
    """Device bytes for a workspace argument (256-byte aligned by the caching allocator)."""
    torch = _torch()
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device or "cuda")


def kv_head_bytes(kv_dtype: int, head_dim: int) -> int:
    return int(_load().gr_kv_head_bytes(kv_dtype, head_dim))


# --------------------------------------------------------------------------- dequant

def _dequant(name: str, per_block: int, block_bytes: int, blocks, out=None):
    torch = _torch()
    n = blocks.numel() // block_bytes
    if out is None:
        out = torch.empty(n * per_block, dtype=torch.float32, device=blocks.device)
    _check(name, getattr(_load(), name)(_ptr(blocks), n, _ptr(out), _stream()))
    return out


def gr_q4k_dequant(blocks, out=None):
    return _dequant("gr_q4k_dequant", 256, 144, blocks, out)


def gr_q6k_dequant(blocks, out=None):
    return _dequant("gr_q6k_dequant", 256, 210, blocks, out)


def gr_q8_0_dequant(blocks, out=None):
    return _dequant("gr_q8_0_dequant", 32, 34, blocks, out)


# --------------------------------------------------------------------------- GEMM

def _gemm(name: str, wblocks, x, n: int, y=None, ws=None):
    torch = _torch()
    b, k = x.shape
    if y is None:
        y = torch.empty((b, n), dtype=torch.float32, device=x.device)
    need = _load().gr_gemm_workspace_size(b, n, k)
    if ws is None:
        ws = workspace(need, x.device)
    _check(name, getattr(_load(), name)(_ptr(wblocks), _ptr(x), _ptr(y), b, n, k, _ptr(ws), ws.numel(), _stream()))
    return y


def gr_q4k_gemm(wblocks, x, n: int, y=None, ws=None):
    """y [B, n] = x [B, K] W^T for a Q4_K matrix of n rows."""
    return _gemm("gr_q4k_gemm", wblocks, x, n, y, ws)


def gr_q6k_gemm(wblocks, x, n: int, y=None, ws=None):
    return _gemm("gr_q6k_gemm", wblocks, x, n, y, ws)


def gr_q5k_gemm(wblocks, x, n: int, y=None, ws=None):
    return _gemm("gr_q5k_gemm", wblocks, x, n, y, ws)


def gr_q8_0_gemm(wblocks, x, n: int, y=None, ws=None):
    return _gemm("gr_q8_0_gemm", wblocks, x, n, y, ws)


GEMM_EPI_STORE, GEMM_EPI_RESIDUAL, GEMM_EPI_SWIGLU = 0, 1, 2


STREAM_READ_WORDS = 2048


def gr_stream_read(buf, out=None):
    """One read-only pass over a device tensor's bytes (the read-ceiling measurement aid);
    returns the per-workgroup int32 checksums (their XOR covers the whole buffer)."""
    torch = _torch()
    if out is None:
        out = torch.empty(STREAM_READ_WORDS, dtype=torch.int32, device=buf.device)
    _check("gr_stream_read", _load().gr_stream_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(out), _stream()))
    return out


def gr_gemm_launch_shape(wtype: int, rows: int, k: int, b: int, epi: int = GEMM_EPI_STORE) -> dict:
    """Which GEMM kernel runs for these sizes, its template parameters and grid.  `kernel`
    is the prefix of the kernel's name as profilers print it."""
    v = [C.c_int() for _ in range(6)]
    _check("gr_gemm_launch_shape", _load().gr_gemm_launch_shape(wtype, rows, k, b, int(epi), *[C.byref(i) for i in v]))
    tl, nt, btn, maxt, grid, block = (i.value for i in v)
    if tl == 2:
        name = f"gemm_mm_kernel<{wtype},"
    elif tl in (3, 5):  # whole-tile tile loop: 2 gate/up pairs, 0 plain store, 1 residual update
        name = f"gemm_tlw_kernel<{2 if nt == 2 else 1 if tl == 5 else 0}>"
    elif tl == 4:
        name = "gemm_kcw_kernel"
    elif tl == 6:  # row-block kernel (gate/up pairs, 17 to 32 rows of Q4_K)
        name = "gemm_rb_kernel"
    else:
        name = f"gemm_tl_kernel<{wtype}, {nt}," if tl else f"gemm_kernel<{wtype}, {nt}, {btn}, {maxt},"
    return {"tile_loop": tl in (1, 3, 5), "whole_tile": tl in (3, 5), "k_chunks": tl == 4, "many_rows": tl == 2,
            "row_block": tl == 6,
            "nt": nt, "btn": btn,
            "maxt": maxt, "grid_threads": grid, "block_threads": block, "kernel": name}


# --------------------------------------------------------------------------- attention

def gr_attn_launch_shape(kv_dtype: int, b: int, n_kv_heads: int, max_tokens: int) -> dict:
    """Launch shape of the decode attention (waves per workgroup, pages per wave, the most
    workgroups of one (row, KV head), grid threads) for rows of up to max_tokens tokens."""
    v = [C.c_int() for _ in range(3)]
    g = C.c_longlong()
    _check("gr_attn_launch_shape", _load().gr_attn_launch_shape(kv_dtype, b, n_kv_heads, max_tokens,
                                                                *[C.byref(i) for i in v], C.byref(g)))
    return {"waves_per_wg": v[0].value, "pages_per_wave": v[1].value, "wg_per_row": v[2].value,
            "grid_threads": g.value, "kernel": f"attn_decode_kernel<{kv_dtype},"}


def attn_meta(n_q_heads, n_kv_heads, head_dim, kv_dtype, num_pages, max_blocks, max_ctx, scale=None) -> AttnMeta:
    return AttnMeta(n_q_heads, n_kv_heads, head_dim, PAGE_SIZE, kv_dtype, num_pages, max_blocks, max_ctx,
                    float(scale if scale is not None else head_dim ** -0.5))


def gr_paged_decode_attn(q, k_pages, v_pages, block_table, ctx_lens, meta: AttnMeta, out=None, ws=None):
    torch = _torch()
    b = q.shape[0]
    if out is None:
        out = torch.empty_like(q)
    need = _load().gr_paged_decode_attn_workspace_size(C.byref(meta), b)
    if ws is None:
        ws = workspace(need, q.device)
    _check("gr_paged_decode_attn",
           _load().gr_paged_decode_attn(_ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(block_table), _ptr(ctx_lens),
                                        _ptr(out), b, C.byref(meta), _ptr(ws), ws.numel(), _stream()))
    return out


def gr_paged_decode_attn_noalloc(q, k_pages, v_pages, block_table, ctx_lens, meta: AttnMeta, out=None):
    """gr_paged_decode_attn with the library's own per-device scratch (no workspace argument)."""
    torch = _torch()
    if out is None:
        out = torch.empty_like(q)
    _check("gr_paged_decode_attn_noalloc",
           _load().gr_paged_decode_attn_noalloc(_ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(block_table),
                                                _ptr(ctx_lens), _ptr(out), q.shape[0], C.byref(meta), _stream()))
    return out


def gr_paged_gather_kv(pages, is_v: bool, block_table, ctx_lens, meta: AttnMeta, out=None):
    torch = _torch()
    b = block_table.shape[0]
    if out is None:
        out = torch.zeros((b, meta.max_ctx, meta.n_kv_heads, meta.head_dim), dtype=torch.float32,
                          device=pages.device)
    _check("gr_paged_gather_kv", _load().gr_paged_gather_kv(_ptr(pages), int(bool(is_v)), _ptr(block_table),
                                                            _ptr(ctx_lens), b, C.byref(meta), _ptr(out), _stream()))
    return out


# --------------------------------------------------------------------------- layer / stack

def layer_cfg(hidden, n_q_heads, n_kv_heads, head_dim, ffn, rms_eps, rope_theta, rope_style, qk_norm,
              kv_dtype) -> LayerCfg:
    return LayerCfg(hidden, n_q_heads, n_kv_heads, head_dim, ffn, float(rms_eps), float(rope_theta), int(rope_style),
                    int(bool(qk_norm)), int(kv_dtype), PAGE_SIZE)


def layer_weights(t: dict) -> LayerWeights:
    """t: dict of device tensors attn_norm, ffn_norm, q_norm?, k_norm?, wq, wk, wv, wo, w_gate, w_up, w_down and
    int types tq, tk, tv, to, tgate, tup, tdown."""
    g = t.get
    return LayerWeights(_ptr(t["attn_norm"]), _ptr(t["ffn_norm"]), _ptr(g("q_norm")), _ptr(g("k_norm")),
                        _ptr(t["wq"]), _ptr(t["wk"]), _ptr(t["wv"]), _ptr(t["wo"]), _ptr(t["w_gate"]),
                        _ptr(t["w_up"]), _ptr(t["w_down"]), t["tq"], t["tk"], t["tv"], t["to"], t["tgate"], t["tup"],
                        t["tdown"])


def decode_layer_workspace_size(cfg: LayerCfg, b: int, max_ctx: int) -> int:
    return int(_load().gr_decode_layer_workspace_size(C.byref(cfg), b, max_ctx))


def gr_decode_layer(cfg: LayerCfg, weights: LayerWeights, k_pages, v_pages, num_pages: int, x, block_table,
                    ctx_lens, max_ctx: int, ws=None):
    b = x.shape[0]
    if ws is None:
        ws = workspace(decode_layer_workspace_size(cfg, b, max_ctx), x.device)
    _check("gr_decode_layer",
           _load().gr_decode_layer(C.byref(cfg), C.byref(weights), _ptr(k_pages), _ptr(v_pages), num_pages, _ptr(x),
                                   _ptr(block_table), block_table.shape[1], _ptr(ctx_lens), max_ctx, b, _ptr(ws),
                                   ws.numel(), _stream()))
    return x


def gr_output_head(x, norm, eps: float, w, wtype: int, vocab: int, logits=None, ws=None):
    torch = _torch()
    b, h = x.shape
    if logits is None:
        logits = torch.empty((b, vocab), dtype=torch.float32, device=x.device)
    if ws is None:
        ws = workspace(_load().gr_output_head_workspace_size(b, h, vocab), x.device)
    _check("gr_output_head", _load().gr_output_head(_ptr(x), _ptr(norm), float(eps), _ptr(w), wtype, _ptr(logits), b,
                                                    h, vocab, _ptr(ws), ws.numel(), _stream()))
    return logits


# --------------------------------------------------------------------------- sampling

SAMPLE_PARAMS_DTYPE = [("temperature", "<f8"), ("top_p", "<f8"), ("u", "<f8"), ("top_k", "<i4"), ("reserved", "<i4")]


def sample_params(temperature, top_p, top_k, u, b: Optional[int] = None, device=None):
    """Device array of gr_sample_params (32 bytes per row) from per-row values or scalars."""
    import numpy as np
    torch = _torch()
    cols = [np.atleast_1d(np.asarray(v)) for v in (temperature, top_p, top_k, u)]
    n = b if b is not None else max(len(c) for c in cols)
    a = np.zeros(n, dtype=SAMPLE_PARAMS_DTYPE)
    a["temperature"] = np.broadcast_to(cols[0], (n,))
    a["top_p"] = np.broadcast_to(cols[1], (n,))
    a["top_k"] = np.broadcast_to(cols[2], (n,))
    a["u"] = np.broadcast_to(cols[3], (n,))
    raw = torch.from_numpy(a.view(np.uint8).copy())
    return raw.to(device or "cuda")


def sample_workspace_size(b: int, vocab: int) -> int:
    return int(_load().gr_sample_workspace_size(b, vocab))


def gr_sample(logits, params, tokens=None, kept=None, ws=None):
    """tokens int32 [B] from f32 logits [B, vocab]; kept (optional int64 [B, 2]) receives (Wk, Wp)."""
    torch = _torch()
    b, vocab = logits.shape
    if params.numel() != 32 * b:
        raise ValueError("params must hold one 32-byte gr_sample_params per row")
    if tokens is None:
        tokens = torch.empty(b, dtype=torch.int32, device=logits.device)
    if ws is None:
        ws = workspace(sample_workspace_size(b, vocab), logits.device)
    _check("gr_sample", _load().gr_sample(_ptr(logits), b, vocab, _ptr(params), _ptr(tokens), _ptr(kept), _ptr(ws),
                                          ws.numel(), _stream()))
    return tokens


def decode_stack_workspace_size(cfg: LayerCfg, b: int, max_ctx: int, vocab: int) -> int:
    return int(_load().gr_decode_stack_workspace_size(C.byref(cfg), b, max_ctx, vocab))


class StackArgs:
    """Host-side argument block of gr_decode_stack kept alive between calls (and graph replays)."""

    def __init__(self, cfg: LayerCfg, layers: Sequence[LayerWeights], k_pools, v_pools):
        n = len(layers)
        self.cfg = cfg
        self.n = n
        self.weights = (LayerWeights * max(n, 1))(*layers)
        self.k = (_p * max(n, 1))(*[_ptr(t) for t in k_pools])
        self.v = (_p * max(n, 1))(*[_ptr(t) for t in v_pools])


def gr_decode_stack(args: StackArgs, num_pages: int, x, block_table, ctx_lens, max_ctx: int, head_norm=None,
                    head_w=None, head_wtype: int = W_Q6_K, vocab: int = 0, logits=None, ws=None):
    b = x.shape[0]
    if ws is None:
        ws = workspace(decode_stack_workspace_size(args.cfg, b, max_ctx, vocab), x.device)
    _check("gr_decode_stack",
           _load().gr_decode_stack(C.byref(args.cfg), args.weights, args.n, args.k, args.v, num_pages, _ptr(x),
                                   _ptr(block_table), block_table.shape[1], _ptr(ctx_lens), max_ctx, b,
                                   _ptr(head_norm), _ptr(head_w), head_wtype, vocab, _ptr(logits), _ptr(ws),
                                   ws.numel(), _stream()))
    return x


def verify_stack_workspace_size(cfg: LayerCfg, b: int, t: int, max_ctx: int, vocab: int) -> int:
    return int(_load().gr_verify_stack_workspace_size(C.byref(cfg), b, t, max_ctx, vocab))


def gr_verify_stack(args: StackArgs, num_pages: int, x, block_table, ctx_lens, max_ctx: int, t: int, head_norm=None,
                    head_w=None, head_wtype: int = W_Q6_K, vocab: int = 0, logits=None, ws=None):
    """T tokens per sequence in one step: x [B*T, hidden] (token j of sequence b in row b*T + j)."""
    rows = x.shape[0]
    if rows % t:
        raise ValueError("x must hold B*T rows")
    b = rows // t
    if ws is None:
        ws = workspace(verify_stack_workspace_size(args.cfg, b, t, max_ctx, vocab), x.device)
    _check("gr_verify_stack",
           _load().gr_verify_stack(C.byref(args.cfg), args.weights, args.n, args.k, args.v, num_pages, _ptr(x),
                                   _ptr(block_table), block_table.shape[1], _ptr(ctx_lens), max_ctx, b, t,
                                   _ptr(head_norm), _ptr(head_w), head_wtype, vocab, _ptr(logits), _ptr(ws),
                                   ws.numel(), _stream()))
    return x


def mixed_stack_workspace_size(cfg: LayerCfg, rows: int, max_pos: int, vocab: int) -> int:
    return int(_load().gr_mixed_stack_workspace_size(C.byref(cfg), rows, max_pos, vocab))


def gr_mixed_stack(args: StackArgs, num_pages: int, x, block_table, row_seq, row_pos, max_pos: int, head_norm=None,
                   head_w=None, head_wtype: int = W_Q6_K, vocab: int = 0, logits=None, ws=None, head_rows=None):
    """Rows placed by (row_seq, row_pos): decode rows, verification runs and prompt chunks in one step.
    With head_rows (device int32), logits are computed for those rows only."""
    rows = x.shape[0]
    if ws is None:
        ws = workspace(mixed_stack_workspace_size(args.cfg, rows, max_pos, vocab), x.device)
    n_head = head_rows.numel() if head_rows is not None else 0
    _check("gr_mixed_stack",
           _load().gr_mixed_stack(C.byref(args.cfg), args.weights, args.n, args.k, args.v, num_pages, _ptr(x),
                                  _ptr(block_table), block_table.shape[1], _ptr(row_seq), _ptr(row_pos), rows, max_pos,
                                  _ptr(head_norm), _ptr(head_w), head_wtype, vocab, _ptr(head_rows), n_head,
                                  _ptr(logits), _ptr(ws), ws.numel(), _stream()))
    return x


def gr_spec_accept(sampled, draft, n_accepted=None):
    """n_accepted int32 [B] from the target's tokens sampled [B, T] and the step's inputs draft [B, T]."""
    torch = _torch()
    b, t = sampled.shape
    if n_accepted is None:
        n_accepted = torch.empty(b, dtype=torch.int32, device=sampled.device)
    _check("gr_spec_accept", _load().gr_spec_accept(_ptr(sampled), _ptr(draft), b, t, _ptr(n_accepted), _stream()))
    return n_accepted


def gr_decode_stack_probed(args: StackArgs, num_pages: int, x, block_table, ctx_lens, max_ctx: int, probe_stage: int,
                           probe_reps: int, ev_begin: Sequence[int], ev_end: Sequence[int], head_norm=None,
                           head_w=None, head_wtype: int = W_Q6_K, vocab: int = 0, logits=None, ws=None):
    """gr_decode_stack with the launches of one stage repeated probe_reps times between
    hipEventRecord calls in each layer; ev_begin / ev_end are raw hipEvent_t handles (ints)."""
    b = x.shape[0]
    if ws is None:
        ws = workspace(decode_stack_workspace_size(args.cfg, b, max_ctx, vocab), x.device)
    eb = (_p * len(ev_begin))(*ev_begin)
    ee = (_p * len(ev_end))(*ev_end)
    _check("gr_decode_stack_probed",
           _load().gr_decode_stack_probed(C.byref(args.cfg), args.weights, args.n, args.k, args.v, num_pages, _ptr(x),
                                          _ptr(block_table), block_table.shape[1], _ptr(ctx_lens), max_ctx, b,
                                          _ptr(head_norm), _ptr(head_w), head_wtype, vocab, _ptr(logits), _ptr(ws),
                                          ws.numel(), _stream(), probe_stage, probe_reps, eb, ee))
    return x
