"""GPU parity of the individual hot-path kernels against the fp64 oracle, through the C ABI.

Bars: dequantization and the page gather are bit-exact; the GEMM and the standalone
attention (fp32 accumulation of exact bf16/f16 hi-lo operands) stay within a
relative L2 error of 1e-4 of the oracle, far inside the layer tolerances.
"""
import dataclasses

import numpy as np
import pytest

import synth
from gpu_util import dev, host, rel_l2, say, torch_cuda

pytestmark = pytest.mark.gpu

KERNEL_TOL = 1e-4


@pytest.fixture(scope="module")
def torch():
    return torch_cuda()


@pytest.fixture(scope="module")
def gr():
    import continuous_quantized_decode_amd as gr
    gr.lib()
    return gr


# ----------------------------------------------------------------------------- dequant

@pytest.mark.parametrize("n_blocks", [1, 16, 37, 1000])
def test_q4k_dequant_bit_exact(torch, gr, orc, n_blocks):
    w = synth.q4k_weight(np.random.default_rng(100 + n_blocks), n_blocks, 256)
    say("q4k dequant", n_blocks)
    got = host(gr.gr_q4k_dequant(dev(w, torch)))
    want = orc.dequant("q4k", w).astype(np.float32)  # exact fp64 value, rounded once
    np.testing.assert_array_equal(got.view(np.uint32), want.view(np.uint32))


@pytest.mark.parametrize("n_blocks", [1, 3, 17, 999])
def test_q6k_dequant_bit_exact(torch, gr, orc, n_blocks):
    # odd block counts put every other block at a 2-mod-4 byte offset
    w = synth.q6k_weight(np.random.default_rng(200 + n_blocks), n_blocks, 256)
    say("q6k dequant", n_blocks)
    got = host(gr.gr_q6k_dequant(dev(w, torch)))
    want = orc.dequant("q6k", w)
    assert np.array_equal(got.astype(np.float64), want)


def test_q8_0_dequant_bit_exact(torch, gr, orc):
    rng = np.random.default_rng(300)
    n = 777
    blk = rng.integers(0, 256, size=(n, 34), dtype=np.uint8)
    blk[:, 0:2] = rng.uniform(1e-3, 1.0, n).astype(np.float16).view(np.uint8).reshape(n, 2)
    say("q8_0 dequant", n)
    got = host(gr.gr_q8_0_dequant(dev(blk, torch)))
    assert np.array_equal(got.astype(np.float64), orc.dequant("q8_0", blk))


def test_handpacked_blocks_on_gpu(torch, gr, orc):
    import json
    import os
    gold = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "handpacked.json")))
    for name, e in sorted(gold.items()):
        raw = np.frombuffer(bytes.fromhex(e["hex"]), np.uint8).copy()
        if e["format"] == "Q5_K":
            # no dequant export for Q5_K: the block as a one-row matrix times one-hot
            # activations (64 per call) gives its 256 weights, to fp32 rounding
            want = orc.dequant("q5k", raw)
            eye = np.eye(256, dtype=np.float32)
            got = np.concatenate([host(gr.gr_q5k_gemm(dev(raw, torch), dev(eye[i:i + 64], torch), 1))[:, 0]
                                  for i in range(0, 256, 64)])
            assert np.abs(got - want).max() <= 1e-6 * np.abs(want).max(), name
            continue
        fn = {"Q4_K": (gr.gr_q4k_dequant, "q4k"), "Q6_K": (gr.gr_q6k_dequant, "q6k"),
              "q8_0": (gr.gr_q8_0_dequant, "q8_0")}[e["format"]]
        got = host(fn[0](dev(raw, torch))).astype(np.float64)
        assert np.array_equal(got, orc.dequant(fn[1], raw)), name


# ----------------------------------------------------------------------------- GEMM

GEMM_CASES = [
    (synth.W_Q4_K, 1, 16, 256),
    (synth.W_Q4_K, 3, 40, 768),      # ragged row tile
    (synth.W_Q4_K, 8, 256, 4096),
    (synth.W_Q4_K, 8, 4096, 4096),   # whole-tile tile loop: one tile per workgroup
    (synth.W_Q4_K, 17, 200, 1024),   # three batch tiles, padded to four
    (synth.W_Q4_K, 32, 512, 2048),
    (synth.W_Q4_K, 64, 64, 512),
    (synth.W_Q6_K, 1, 16, 256),
    (synth.W_Q6_K, 5, 48, 768),      # odd blocks per row: 2-byte aligned blocks
    (synth.W_Q6_K, 8, 1024, 3072),
    (synth.W_Q6_K, 8, 4096, 14336),
    (synth.W_Q6_K, 12, 100, 1280),
    (synth.W_Q6_K, 32, 256, 1024),
    (synth.W_Q6_K, 32, 256, 4096),   # several super-blocks per wave with four batch tiles
    (synth.W_Q6_K, 16, 256, 12288),
    (synth.W_Q6_K, 64, 128, 14336),
    (synth.W_Q4_K, 64, 256, 14336),
    # 17 to 32 rows of Q4_K at K of two, four and seven ranges of the row-block kernel's
    # (which takes only the gate/up pairs: the plain stores keep the split-K kernel)
    (synth.W_Q4_K, 32, 6144, 4096),
    (synth.W_Q4_K, 24, 1000, 4096),
    (synth.W_Q4_K, 20, 4096, 3072),
    (synth.W_Q4_K, 17, 2000, 5120),
    (synth.W_Q4_K, 32, 300, 14336),
    # tile-loop kernel (at least two tile groups per CU, one batch tile, K <= 4096)
    (synth.W_Q4_K, 8, 8200, 4096),   # 513 tiles, the last ragged (whole-tile tile loop, two or three per workgroup)
    (synth.W_Q4_K, 7, 6144, 4096),   # the QKV shape: 384 tiles, one or two per workgroup
    (synth.W_Q6_K, 5, 9000, 1280),   # 2-byte aligned rows, waves of two and one super-blocks
    (synth.W_Q6_K, 8, 8192, 4096),
    (synth.W_Q4_K, 1, 16384, 256),   # one super-block: too few waves for the tile loop
    (synth.W_Q4_K, 8, 16384, 256),   # the same at 8 rows (every row's outputs written)
    (synth.W_Q6_K, 6, 9000, 512),
    (synth.W_Q4_K, 8, 9000, 768),    # three super-blocks: the smallest tile-loop K
    (synth.W_Q4_K, 12, 9000, 2048),  # tile loop with two batch tiles (ragged rows and tiles)
    (synth.W_Q6_K, 16, 8200, 4096),
    (synth.W_Q6_K, 10, 9000, 1792),  # 2-byte aligned rows, seven super-blocks
    # Q5_K and Q8_0 rows (split-K kernel only): every batch-tile count, ragged rows
    (synth.W_Q5_K, 1, 16, 256),
    (synth.W_Q5_K, 2, 40, 768),
    (synth.W_Q5_K, 4, 1000, 4096),
    (synth.W_Q5_K, 7, 4096, 4096),
    (synth.W_Q5_K, 13, 300, 1280),
    (synth.W_Q5_K, 32, 256, 2048),
    (synth.W_Q5_K, 64, 96, 14336),
    (synth.W_Q5_K, 8, 9000, 1024),   # many tiles: no tile-loop kernel for this type
    (synth.W_Q8_0, 1, 16, 256),
    (synth.W_Q8_0, 3, 40, 768),
    (synth.W_Q8_0, 4, 1000, 4096),
    (synth.W_Q8_0, 8, 4096, 4096),
    (synth.W_Q8_0, 9, 300, 1280),
    (synth.W_Q8_0, 24, 256, 2048),
    (synth.W_Q8_0, 64, 96, 14336),
    (synth.W_Q8_0, 8, 9000, 1024),
]

GEMM_FN = {synth.W_Q4_K: "gr_q4k_gemm", synth.W_Q6_K: "gr_q6k_gemm", synth.W_Q5_K: "gr_q5k_gemm",
           synth.W_Q8_0: "gr_q8_0_gemm"}


@pytest.mark.parametrize("wtype,b,n,k", GEMM_CASES)
def test_gemm_matches_oracle(torch, gr, orc, wtype, b, n, k):
    rng = np.random.default_rng(1000 + b * 7 + n + k)
    w = synth.weight(rng, wtype, n, k)
    x = rng.standard_normal((b, k), dtype=np.float32)
    say("gemm", wtype, b, n, k, gr.gr_gemm_launch_shape(wtype, n, k, b)["kernel"])
    fn = getattr(gr, GEMM_FN[wtype])
    got = host(fn(dev(w, torch), dev(x, torch), n))
    want = orc.gemm(wtype, w, x, n, k)
    err = rel_l2(got, want)
    say("  rel_l2", err)
    assert err <= KERNEL_TOL


def test_gemm_large_activation_range(torch, gr, orc):
    """bf16 hi/lo keeps the full fp32 range: activations up to 1e6 and down to 1e-6."""
    rng = np.random.default_rng(7)
    n, k, b = 64, 1024, 4
    w = synth.q4k_weight(rng, n, k)
    x = (rng.standard_normal((b, k)) * 10.0 ** rng.uniform(-6, 6, (b, k))).astype(np.float32)
    got = host(gr.gr_q4k_gemm(dev(w, torch), dev(x, torch), n))
    assert rel_l2(got, orc.gemm(synth.W_Q4_K, w, x, n, k)) <= KERNEL_TOL


@pytest.mark.parametrize("wtype", [synth.W_Q5_K, synth.W_Q8_0])
def test_gemm_large_activation_range_q5_q8(torch, gr, orc, wtype):
    """The Q5_K / Q8_0 decoders under activations from 1e-6 to 1e6 (Q8_0's -2304 start and
    the two code MFMAs cancel exactly only if every product is exact)."""
    rng = np.random.default_rng(17 + wtype)
    n, k, b = 80, 2048, 3
    w = synth.weight(rng, wtype, n, k)
    x = (rng.standard_normal((b, k)) * 10.0 ** rng.uniform(-6, 6, (b, k))).astype(np.float32)
    got = host(getattr(gr, GEMM_FN[wtype])(dev(w, torch), dev(x, torch), n))
    assert rel_l2(got, orc.gemm(wtype, w, x, n, k)) <= KERNEL_TOL


@pytest.mark.parametrize("wtype", [synth.W_Q4_K, synth.W_Q5_K, synth.W_Q6_K, synth.W_Q8_0])
def test_output_head_each_weight_type(torch, gr, orc, wtype):
    """The output head (final RMSNorm fused into the GEMM) over a vocabulary of 5000 rows
    in each weight format, at B = 5."""
    rng = np.random.default_rng(23 + wtype)
    h, vocab, b = 1024, 5000, 5
    x = synth.activations(rng, b, h)
    norm = (1.0 + 0.1 * rng.standard_normal(h)).astype(np.float32)
    w = synth.weight(rng, wtype, vocab, h)
    say("head", wtype, b, vocab, h)
    got = host(gr.gr_output_head(dev(x, torch), dev(norm, torch), 1e-6, dev(w, torch), wtype, vocab))
    err = rel_l2(got, orc.output_head(x, norm, 1e-6, w, wtype, vocab))
    say("  rel_l2", err)
    assert err <= KERNEL_TOL


def test_gemm_rows_independent(torch, gr):
    """Batched rows equal the same rows computed alone (the pages' batched-service check)."""
    rng = np.random.default_rng(8)
    n, k = 512, 2048
    w = dev(synth.q4k_weight(rng, n, k), torch)
    x = rng.standard_normal((8, k), dtype=np.float32)
    full = host(gr.gr_q4k_gemm(w, dev(x, torch), n))
    for r in (0, 5):
        one = host(gr.gr_q4k_gemm(w, dev(x[r:r + 1], torch), n))
        assert rel_l2(one[0], full[r]) <= KERNEL_TOL


# ----------------------------------------------------------------------------- attention

def _attn_case(kv_dtype, d, hq, hkv, ctx, seed, pool_kind="exact"):
    wl = dataclasses.replace(synth.WORKLOADS["tiny"], kv_dtype=kv_dtype, head_dim=d, n_q_heads=hq, n_kv_heads=hkv,
                             batch=len(ctx), pool_kind=pool_kind, seed=seed)
    c = np.asarray(ctx, np.int32)
    kv = synth.kv_state(wl, c, n_layers=1, extra_slot=False)
    q = synth.attn_query(np.random.default_rng(seed), len(ctx), hq, d)
    return wl, c, kv, q


ATTN_CASES = [
    (synth.KV_F16, 128, 8, 2, [1, 15, 16, 17, 300]),
    (synth.KV_F16, 128, 32, 8, [1000, 64, 4097]),
    (synth.KV_F16, 64, 4, 2, [128, 33]),
    (synth.KV_F32, 64, 4, 2, [128, 1, 250]),
    (synth.KV_F32, 128, 16, 8, [77, 512]),
    (synth.KV_Q8_0, 128, 32, 8, [2000, 16, 5]),
    (synth.KV_Q8_0, 64, 8, 1, [31, 700]),
    (synth.KV_F16, 128, 24, 8, [40, 3]),   # GQA ratio 3
]


@pytest.mark.parametrize("kv_dtype,d,hq,hkv,ctx", ATTN_CASES)
def test_paged_attention_matches_oracle(torch, gr, orc, kv_dtype, d, hq, hkv, ctx):
    wl, c, kv, q = _attn_case(kv_dtype, d, hq, hkv, ctx, seed=len(ctx) + d + hq)
    pm = kv.pages
    meta = gr.attn_meta(hq, hkv, d, kv_dtype, pm.num_pages, pm.max_blocks, int(c.max()))
    say("attn", kv_dtype, d, hq, hkv, ctx)
    got = host(gr.gr_paged_decode_attn(dev(q, torch), dev(kv.k_pools[0], torch), dev(kv.v_pools[0], torch),
                                       dev(pm.block_table, torch), dev(c, torch), meta))
    want = orc.paged_attention(q, kv.k_pools[0], kv.v_pools[0], kv_dtype, pm.block_table, c, hkv)
    assert np.isfinite(got).all()
    err = rel_l2(got, want)
    say("  rel_l2", err)
    assert err <= KERNEL_TOL


def test_paged_attention_page_permutation_is_bitwise_invariant(torch, gr):
    wl, c, kv, q = _attn_case(synth.KV_F16, 128, 8, 2, [333, 40], seed=5)
    pm = kv.pages
    meta = gr.attn_meta(8, 2, 128, synth.KV_F16, pm.num_pages, pm.max_blocks, int(c.max()))
    base = host(gr.gr_paged_decode_attn(dev(q, torch), dev(kv.k_pools[0], torch), dev(kv.v_pools[0], torch),
                                        dev(pm.block_table, torch), dev(c, torch), meta))
    perm = np.random.default_rng(6).permutation(pm.num_pages)
    kp, vp = np.empty_like(kv.k_pools[0]), np.empty_like(kv.v_pools[0])
    kp[perm], vp[perm] = kv.k_pools[0], kv.v_pools[0]
    bt = np.where(pm.block_table >= 0, perm[np.maximum(pm.block_table, 0)], -1).astype(np.int32)
    moved = host(gr.gr_paged_decode_attn(dev(q, torch), dev(kp, torch), dev(vp, torch), dev(bt, torch),
                                         dev(c, torch), meta))
    assert np.array_equal(base, moved)


@pytest.mark.parametrize("kv_dtype,d", [(synth.KV_F32, 64), (synth.KV_F16, 128), (synth.KV_Q8_0, 128),
                                        (synth.KV_Q8_0, 64)])
def test_page_gather_bit_exact(torch, gr, orc, kv_dtype, d):
    wl, c, kv, _ = _attn_case(kv_dtype, d, 4, 2, [1, 16, 17, 90], seed=11, pool_kind="fill90")
    pm = kv.pages
    meta = gr.attn_meta(4, 2, d, kv_dtype, pm.num_pages, pm.max_blocks, int(c.max()))
    for is_v, pool in ((False, kv.k_pools[0]), (True, kv.v_pools[0])):
        got = host(gr.gr_paged_gather_kv(dev(pool, torch), is_v, dev(pm.block_table, torch), dev(c, torch), meta))
        want = orc.gather_kv(pool, kv_dtype, is_v, 2, d, pm.block_table, c)
        off = 0
        for b, n in enumerate(c):
            assert np.array_equal(got[b, :n].astype(np.float64), want[off:off + n]), (is_v, b)
            off += n


@pytest.mark.parametrize("nbytes", [16, 8192 * 3 + 48, (1 << 24) + 16 * 7])
def test_stream_read_checksum(torch, gr, nbytes):
    """The read-ceiling kernel reads every 16-byte unit once: its XOR of each unit's
    first and last dword equals numpy's (sizes below one step, ragged, and many steps)."""
    a = np.random.default_rng(nbytes).integers(0, 2 ** 32, size=nbytes // 4, dtype=np.uint32)
    want = np.bitwise_xor.reduce(a.reshape(-1, 4)[:, 0] ^ a.reshape(-1, 4)[:, 3])
    got = host(gr.gr_stream_read(dev(a.view(np.int32), torch))).view(np.uint32)
    assert int(np.bitwise_xor.reduce(got)) == int(want)
