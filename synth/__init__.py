"""Seeded synthetic inputs for the continuous-batched quantized decode step.

This module is shared by the tests, the bench and the smoke check.  It only
draws random numbers and writes them into the storage formats the decode step
consumes (GGUF Q4_K / Q6_K super-blocks, paged KV pools, block tables).  It
holds none of the method's arithmetic: no dequantization, no quantizer, no
norm, rope, GEMM or attention.  Both the HIP path and the CPU oracle receive
exactly the buffers produced here.

Workload shapes follow the five workloads the decode study is quoted on
(a tiny single layer, a Qwen3-0.6B-shaped stack, a Llama-3-8B-shaped stack, a
Qwen3-8B-shaped stack, and a long-context Llama-3-8B layer).  Weight formats
follow the public GGUF block layouts; pages hold 16 tokens (tinyllm page,
"Known limitations": 16-token pages).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional, Tuple

import numpy as np

# GGUF tensor type ids (public GGUF enumeration) used as weight-type tags.
W_Q8_0 = 8
W_Q4_K = 12
W_Q5_K = 13
W_Q6_K = 14

KV_F32 = 0
KV_F16 = 1
KV_Q8_0 = 2

ROPE_NEOX = 0
ROPE_NORM = 1

PAGE = 16
Q4K_BYTES = 144
Q5K_BYTES = 176
Q6K_BYTES = 210
Q8_0_BYTES = 34
QK = 256  # weights per K-quant super-block
Q8_BLOCK = 32  # q8_0 block length along head_dim

F16_NAN_BITS = 0x7E00


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    index: int
    n_layers: int
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    rms_eps: float
    rope_theta: float
    rope_style: int
    qk_norm: bool
    kv_dtype: int
    batch: int
    ctx_kind: str  # "fixed", "uniform", "loguniform"
    ctx_lo: int
    ctx_hi: int
    pool_kind: str  # "exact" (exactly the needed pages, shuffled) or "fill90"
    w_down: int
    w_other: int = W_Q4_K
    vocab: int = 0  # 0: no output head
    w_head: int = W_Q6_K
    seed: int = 0

    @property
    def q_dim(self) -> int:
        return self.n_q_heads * self.head_dim

    @property
    def kv_dim(self) -> int:
        return self.n_kv_heads * self.head_dim


WORKLOADS: Dict[str, Workload] = {
    # Tiny single decode layer, CPU-seconds.
    "tiny": Workload("tiny", 0, 1, 256, 4, 2, 64, 768, 1e-6, 1e4, ROPE_NEOX, False,
                     KV_F32, 1, "fixed", 128, 128, "exact", W_Q4_K),
    # Qwen3-0.6B-shaped stack.
    "qwen3_0p6b": Workload("qwen3_0p6b", 1, 28, 1024, 16, 8, 128, 3072, 1e-6, 1e6, ROPE_NEOX, True,
                           KV_F16, 8, "uniform", 64, 1024, "exact", W_Q6_K),
    # Llama-3-8B-shaped stack with the Q6_K output head.
    "llama3_8b": Workload("llama3_8b", 2, 32, 4096, 32, 8, 128, 14336, 1e-5, 5e5, ROPE_NORM, False,
                          KV_F16, 8, "uniform", 256, 4096, "exact", W_Q6_K, vocab=128256),
    # Qwen3-8B-shaped stack, q8_0 KV, fragmented pool filled to 90 %.
    "qwen3_8b": Workload("qwen3_8b", 3, 36, 4096, 32, 8, 128, 12288, 1e-6, 1e6, ROPE_NEOX, True,
                         KV_Q8_0, 32, "loguniform", 512, 8192, "fill90", W_Q6_K),
    # Long-context attention stress: one Llama-3-8B layer, B=64, q8_0 KV.
    "longctx": Workload("longctx", 4, 1, 4096, 32, 8, 128, 14336, 1e-5, 5e5, ROPE_NORM, False,
                        KV_Q8_0, 64, "uniform", 4096, 32768, "fill90", W_Q4_K),
}


def rng_for(w: Workload, *key: int) -> np.random.Generator:
    """Independent stream per (workload, key...) from SeedSequence(seed)."""
    ss = np.random.SeedSequence(entropy=w.seed, spawn_key=(w.index,) + tuple(int(k) for k in key))
    return np.random.default_rng(ss)


def rng_plain(seed: int, *key: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence(entropy=seed, spawn_key=tuple(int(k) for k in key)))


# --------------------------------------------------------------------------------------------
# weights
# --------------------------------------------------------------------------------------------

_CHUNK = 32 << 20  # bytes per independent random stream when filling large buffers
_POOL = None


def _pool():
    global _POOL
    if _POOL is None:
        import concurrent.futures
        import os
        _POOL = concurrent.futures.ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1))
    return _POOL


def random_bytes(ss: np.random.SeedSequence, nbytes: int) -> np.ndarray:
    """nbytes uniform random bytes; chunk i comes from ss.spawn()[i], so the result does
    not depend on how many threads fill it."""
    out = np.empty(nbytes, dtype=np.uint8)
    n_chunks = max(1, (nbytes + _CHUNK - 1) // _CHUNK)
    kids = ss.spawn(n_chunks)

    def fill(i):
        s, e = i * _CHUNK, min(nbytes, (i + 1) * _CHUNK)
        out[s:e] = np.frombuffer(np.random.default_rng(kids[i]).bytes(e - s), dtype=np.uint8)

    list(_pool().map(fill, range(n_chunks)))
    return out


def random_normal_f32(ss: np.random.SeedSequence, n: int) -> np.ndarray:
    out = np.empty(n, dtype=np.float32)
    per = _CHUNK // 4
    n_chunks = max(1, (n + per - 1) // per)
    kids = ss.spawn(n_chunks)

    def fill(i):
        s, e = i * per, min(n, (i + 1) * per)
        out[s:e] = np.random.default_rng(kids[i]).standard_normal(e - s, dtype=np.float32)

    list(_pool().map(fill, range(n_chunks)))
    return out


def _seq(rng: np.random.Generator) -> np.random.SeedSequence:
    return np.random.SeedSequence(rng.integers(0, 2**63))


def _f16_uniform_bits(rng: np.random.Generator, n: int, lo: float, hi: float) -> np.ndarray:
    return rng.uniform(lo, hi, size=n).astype(np.float16).view(np.uint16)


def q4k_weight(rng: np.random.Generator, n_rows: int, k: int) -> np.ndarray:
    """Random Q4_K matrix: n_rows rows of k/256 super-blocks (144 B each), row-major.

    Quants and the 12 packed scale/min bytes are uniform random bytes (the 12-byte
    packing is a bijection onto sixteen 6-bit values, so every 6-bit scale and min
    is uniform); d and dmin are fp16 draws of U(1e-3, 1e-2).
    """
    assert k % QK == 0
    nb = k // QK
    out = random_bytes(_seq(rng), n_rows * nb * Q4K_BYTES).reshape(n_rows, nb, Q4K_BYTES)
    dd = _f16_uniform_bits(rng, n_rows * nb * 2, 1e-3, 1e-2).reshape(n_rows, nb, 2)
    out[:, :, 0:4] = dd.view(np.uint8).reshape(n_rows, nb, 4)
    return out.reshape(n_rows, nb * Q4K_BYTES)


def q6k_weight(rng: np.random.Generator, n_rows: int, k: int) -> np.ndarray:
    """Random Q6_K matrix: ql, qh and the int8 scales are uniform random bytes,
    d is an fp16 draw of U(1e-3, 1e-2) stored in the last two bytes of each block."""
    assert k % QK == 0
    nb = k // QK
    out = random_bytes(_seq(rng), n_rows * nb * Q6K_BYTES).reshape(n_rows, nb, Q6K_BYTES)
    d = _f16_uniform_bits(rng, n_rows * nb, 1e-3, 1e-2).reshape(n_rows, nb, 1)
    out[:, :, 208:210] = d.view(np.uint8).reshape(n_rows, nb, 2)
    return out.reshape(n_rows, nb * Q6K_BYTES)


def q5k_weight(rng: np.random.Generator, n_rows: int, k: int) -> np.ndarray:
    """Random Q5_K matrix: n_rows rows of k/256 super-blocks (176 B each): uniform random
    quant, high-bit and packed scale/min bytes; d and dmin fp16 draws of U(1e-3, 1e-2)."""
    assert k % QK == 0
    nb = k // QK
    out = random_bytes(_seq(rng), n_rows * nb * Q5K_BYTES).reshape(n_rows, nb, Q5K_BYTES)
    dd = _f16_uniform_bits(rng, n_rows * nb * 2, 1e-3, 1e-2).reshape(n_rows, nb, 2)
    out[:, :, 0:4] = dd.view(np.uint8).reshape(n_rows, nb, 4)
    return out.reshape(n_rows, nb * Q5K_BYTES)


def q8_0_weight(rng: np.random.Generator, n_rows: int, k: int) -> np.ndarray:
    """Random Q8_0 matrix: n_rows rows of k/32 blocks (34 B each): uniform random int8
    codes (all 256 values) and fp16 scales d of U(1e-4, 1e-3)."""
    assert k % QK == 0
    nb = k // Q8_BLOCK
    out = random_bytes(_seq(rng), n_rows * nb * Q8_0_BYTES).reshape(n_rows, nb, Q8_0_BYTES)
    d = _f16_uniform_bits(rng, n_rows * nb, 1e-4, 1e-3).reshape(n_rows, nb, 1)
    out[:, :, 0:2] = d.view(np.uint8).reshape(n_rows, nb, 2)
    return out.reshape(n_rows, nb * Q8_0_BYTES)


def weight(rng: np.random.Generator, wtype: int, n_rows: int, k: int) -> np.ndarray:
    if wtype == W_Q4_K:
        return q4k_weight(rng, n_rows, k)
    if wtype == W_Q6_K:
        return q6k_weight(rng, n_rows, k)
    if wtype == W_Q5_K:
        return q5k_weight(rng, n_rows, k)
    if wtype == W_Q8_0:
        return q8_0_weight(rng, n_rows, k)
    raise ValueError(f"unknown weight type {wtype}")


def norm_gain(rng: np.random.Generator, n: int) -> np.ndarray:
    return rng.uniform(0.5, 1.5, size=n).astype(np.float32)


def activations(rng: np.random.Generator, b: int, n: int) -> np.ndarray:
    return rng.standard_normal((b, n), dtype=np.float32)


@dataclasses.dataclass
class LayerWeights:
    attn_norm: np.ndarray
    ffn_norm: np.ndarray
    q_norm: Optional[np.ndarray]
    k_norm: Optional[np.ndarray]
    wq: np.ndarray
    wk: np.ndarray
    wv: np.ndarray
    wo: np.ndarray
    w_gate: np.ndarray
    w_up: np.ndarray
    w_down: np.ndarray
    tq: int
    tk: int
    tv: int
    to: int
    tgate: int
    tup: int
    tdown: int


def layer_weights(w: Workload, layer: int) -> LayerWeights:
    r = lambda t: rng_for(w, 1, layer, t)  # noqa: E731
    H, F, qd, kvd = w.hidden, w.ffn, w.q_dim, w.kv_dim
    t = w.w_other
    return LayerWeights(
        attn_norm=norm_gain(r(0), H),
        ffn_norm=norm_gain(r(1), H),
        q_norm=norm_gain(r(2), w.head_dim) if w.qk_norm else None,
        k_norm=norm_gain(r(3), w.head_dim) if w.qk_norm else None,
        wq=weight(r(4), t, qd, H),
        wk=weight(r(5), t, kvd, H),
        wv=weight(r(6), t, kvd, H),
        wo=weight(r(7), t, H, qd),
        w_gate=weight(r(8), t, F, H),
        w_up=weight(r(9), t, F, H),
        w_down=weight(r(10), w.w_down, H, F),
        tq=t, tk=t, tv=t, to=t, tgate=t, tup=t, tdown=w.w_down,
    )


def head_weights(w: Workload) -> Tuple[np.ndarray, np.ndarray]:
    """(final norm gain, output head matrix) for workloads with a head."""
    assert w.vocab > 0
    return norm_gain(rng_for(w, 2, 0), w.hidden), weight(rng_for(w, 2, 1), w.w_head, w.vocab, w.hidden)


def input_x(w: Workload, batch: Optional[int] = None) -> np.ndarray:
    return activations(rng_for(w, 3, 0), batch or w.batch, w.hidden)


# --------------------------------------------------------------------------------------------
# contexts, block tables and paged KV pools
# --------------------------------------------------------------------------------------------

def ctx_lens(w: Workload, batch: Optional[int] = None) -> np.ndarray:
    """Tokens already cached per row (the new token is written at this position)."""
    b = batch or w.batch
    rng = rng_for(w, 4, 0)
    if w.ctx_kind == "fixed":
        c = np.full(b, w.ctx_lo, dtype=np.int64)
    elif w.ctx_kind == "uniform":
        c = rng.integers(w.ctx_lo, w.ctx_hi + 1, size=b)
    elif w.ctx_kind == "loguniform":
        u = rng.uniform(math.log(w.ctx_lo), math.log(w.ctx_hi + 1), size=b)
        c = np.clip(np.floor(np.exp(u)), w.ctx_lo, w.ctx_hi).astype(np.int64)
    else:
        raise ValueError(w.ctx_kind)
    return c.astype(np.int32)


@dataclasses.dataclass
class PageMap:
    block_table: np.ndarray  # int32 [B, max_blocks]; -1 where unused
    num_pages: int
    max_blocks: int
    used_pages: np.ndarray  # sorted physical ids that hold some row's tokens


def page_map(rng: np.random.Generator, ctx: np.ndarray, pool_kind: str, max_ctx: Optional[int] = None,
             extra_slot=True) -> PageMap:
    """Allocate pages for every row: ceil((ctx+n)/16) pages when the step appends n tokens
    (extra_slot: True for one, an int for several, False for none).  "exact" pools hold
    exactly the needed pages in a random order; "fill90" pools have ceil(needed/0.9) pages
    with the used ones a random subset in random order (a fragmented pool)."""
    n_extra = int(extra_slot)
    tok = ctx.astype(np.int64) + n_extra
    per_row = (tok + PAGE - 1) // PAGE
    needed = int(per_row.sum())
    mc = int(max_ctx if max_ctx is not None else int(ctx.max(initial=0)))
    max_blocks = max(1, (mc + n_extra + PAGE - 1) // PAGE, int(per_row.max(initial=1)))
    if pool_kind == "exact":
        num_pages = max(needed, 1)
        phys = rng.permutation(num_pages)[:needed]
    elif pool_kind == "fill90":
        num_pages = max(int(math.ceil(needed / 0.9)), 1)
        phys = rng.permutation(num_pages)[:needed]
    else:
        raise ValueError(pool_kind)
    bt = np.full((len(ctx), max_blocks), -1, dtype=np.int32)
    off = 0
    for b, n in enumerate(per_row):
        bt[b, :n] = phys[off:off + n]
        off += n
    return PageMap(bt, num_pages, max_blocks, np.sort(phys))


def kv_page_bytes(kv_dtype: int, n_kv_heads: int, head_dim: int) -> int:
    """Bytes of one page (16 tokens, all KV heads) of one pool."""
    return n_kv_heads * head_bytes(kv_dtype, head_dim)


def head_bytes(kv_dtype: int, head_dim: int) -> int:
    if kv_dtype == KV_F32:
        return PAGE * head_dim * 4
    if kv_dtype == KV_F16:
        return PAGE * head_dim * 2
    if kv_dtype == KV_Q8_0:
        return PAGE * head_dim + PAGE * (head_dim // Q8_BLOCK) * 2
    raise ValueError(kv_dtype)


def _fill_pool(rng: np.random.Generator, kv_dtype: int, n_pages: int, hkv: int, d: int) -> np.ndarray:
    """Pool bytes [n_pages, page_bytes] in storage format.

    f32 / f16: N(0,1) cast to the storage type.  q8_0: int8 codes uniform on
    [-127, 127] and fp16 scales U(0.011, 0.016), so dequantized values have a
    standard deviation near 1; codes and scales are drawn directly in storage form.
    """
    pb = kv_page_bytes(kv_dtype, hkv, d)
    if kv_dtype == KV_F32:
        return random_normal_f32(_seq(rng), n_pages * pb // 4).view(np.uint8).reshape(n_pages, pb)
    if kv_dtype == KV_F16:
        return random_normal_f32(_seq(rng), n_pages * pb // 2).astype(np.float16).view(np.uint8).reshape(n_pages, pb)
    hb = head_bytes(kv_dtype, d)
    out = random_bytes(_seq(rng), n_pages * pb).reshape(n_pages, hkv, hb)
    codes = out[:, :, :PAGE * d].view(np.int8)
    np.maximum(codes, -127, out=codes)
    sc = rng.uniform(0.011, 0.016, size=(n_pages, hkv, PAGE * (d // Q8_BLOCK))).astype(np.float16)
    out[:, :, PAGE * d:] = sc.view(np.uint8)
    return out.reshape(n_pages, pb)


def _poison_slots(pool: np.ndarray, kv_dtype: int, is_v: bool, hkv: int, d: int, page: int, slots: List[int]) -> None:
    """Make the given token slots of one page decode to NaN (every head, every element)."""
    if not slots:
        return
    hb = head_bytes(kv_dtype, d)
    for h in range(hkv):
        base = h * hb
        if kv_dtype in (KV_F32, KV_F16):
            es = 4 if kv_dtype == KV_F32 else 2
            nan = np.array([np.nan], dtype=np.float32 if es == 4 else np.float16).view(np.uint8)
            view = pool[page, base:base + hb].reshape(-1, es)  # element view
            for t in slots:
                idx = (np.arange(d) * PAGE + t) if is_v else (t * d + np.arange(d))
                view[idx] = nan
        else:
            sc = pool[page, base + PAGE * d: base + hb].view(np.uint16).reshape(PAGE, d // Q8_BLOCK)
            for t in slots:
                sc[t, :] = F16_NAN_BITS


def _poison_pages(pool: np.ndarray, kv_dtype: int, hkv: int, d: int, pages: np.ndarray) -> None:
    """Make whole pages decode to NaN."""
    if len(pages) == 0:
        return
    if kv_dtype == KV_F32:
        pool[pages] = np.full(pool.shape[1] // 4, np.nan, dtype=np.float32).view(np.uint8)
    elif kv_dtype == KV_F16:
        pool[pages] = np.full(pool.shape[1] // 2, np.nan, dtype=np.float16).view(np.uint8)
    else:
        hb = head_bytes(kv_dtype, d)
        nsc = PAGE * (d // Q8_BLOCK)
        nanbytes = np.full(nsc, F16_NAN_BITS, dtype=np.uint16).view(np.uint8)
        for h in range(hkv):
            pool[pages, h * hb + PAGE * d: (h + 1) * hb] = nanbytes


@dataclasses.dataclass
class KVState:
    kv_dtype: int
    n_kv_heads: int
    head_dim: int
    pages: PageMap
    k_pools: List[np.ndarray]  # per layer: uint8 [num_pages, page_bytes]
    v_pools: List[np.ndarray]


def kv_state(w: Workload, ctx: np.ndarray, n_layers: Optional[int] = None, extra_slot=True,
             max_ctx: Optional[int] = None, poison: bool = True, seed_key: int = 0) -> KVState:
    """Paged K/V pools for every layer plus the shared block table.

    Layout per pool page: for each KV head, K is token-major [16][D] and V is
    dim-major [D][16]; q8_0 heads store the int8 codes in that order followed by
    fp16 scales [16 tokens][D/32].  Unused pages and unused slots (including the
    slots the step appends into: one with extra_slot=True, n with an int) decode to NaN
    when `poison` is set.
    """
    L = n_layers if n_layers is not None else w.n_layers
    rng = rng_for(w, 5, seed_key)
    pm = page_map(rng, ctx, w.pool_kind, max_ctx=max_ctx, extra_slot=extra_slot)
    hkv, d = w.n_kv_heads, w.head_dim
    kp, vp = [], []
    used = np.zeros(pm.num_pages, dtype=bool)
    used[pm.used_pages] = True
    for layer in range(L):
        for is_v, lst in ((False, kp), (True, vp)):
            pool = _fill_pool(rng_for(w, 6, seed_key, layer, int(is_v)), w.kv_dtype, pm.num_pages, hkv, d)
            if poison:
                _poison_pages(pool, w.kv_dtype, hkv, d, np.nonzero(~used)[0])
                n_extra = int(extra_slot)
                for b, c in enumerate(ctx):
                    c = int(c)
                    # positions c .. end of the row's last page are not cached yet
                    n_pg = (c + n_extra + PAGE - 1) // PAGE
                    for pg in range(c // PAGE, n_pg):
                        first = max(c - pg * PAGE, 0)
                        _poison_slots(pool, w.kv_dtype, is_v, hkv, d, int(pm.block_table[b, pg]),
                                      list(range(first, PAGE)))
            lst.append(pool)
    return KVState(w.kv_dtype, hkv, d, pm, kp, vp)


def attn_query(rng: np.random.Generator, b: int, hq: int, d: int) -> np.ndarray:
    """Standalone attention query ~ N(0,1) (scores of std ~1 at D=128 after 1/sqrt(D))."""
    return rng.standard_normal((b, hq, d), dtype=np.float32)


def sample_logits(rng: np.random.Generator, b: int, vocab: int, sigma: float = 2.5, spikes: int = 8,
                  spike_lo: float = 4.0, spike_hi: float = 12.0) -> np.ndarray:
    """Logits for the sampler: N(0, sigma) over the vocabulary plus `spikes` tokens per row
    lifted by U(spike_lo, spike_hi) (a few likely tokens above a broad tail, the shape of a
    language model's next-token logits).  float32 [b, vocab]."""
    x = rng.normal(0.0, sigma, (b, vocab)).astype(np.float32)
    for r in range(b):
        if spikes:
            idx = rng.choice(vocab, min(spikes, vocab), replace=False)
            x[r, idx] += rng.uniform(spike_lo, spike_hi, len(idx)).astype(np.float32)
    return x


def sample_uniforms(rng: np.random.Generator, b: int) -> np.ndarray:
    """The per-row uniform draws in [0, 1) the sampler consumes (float64)."""
    return rng.random(b)
