"""The C-ABI library loads and exports every function include/gr.h declares (no GPU)."""
import ctypes
import os
import re

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gr.h")
LIB = os.path.join(ROOT, "continuous_quantized_decode_amd", "libgr.so")


def declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(gr_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_the_hot_path_calls():
    names = declared()
    for n in ("gr_q4k_gemm", "gr_q6k_gemm", "gr_paged_decode_attn", "gr_decode_layer", "gr_decode_stack",
              "gr_q4k_dequant", "gr_q6k_dequant", "gr_q8_0_dequant", "gr_paged_gather_kv", "gr_output_head"):
        assert n in names


def test_library_exports_every_declared_symbol():
    assert os.path.exists(LIB), "build first: python -m continuous_quantized_decode_amd.build"
    lib = ctypes.CDLL(LIB)
    missing = [n for n in declared() if not hasattr(lib, n)]
    assert not missing, missing


def test_binding_lists_match_header():
    import continuous_quantized_decode_amd as gr
    assert sorted(gr.EXPORTED) == declared()


def test_host_side_checks_without_gpu():
    """Calls that fail a host check return their status before touching the device."""
    import continuous_quantized_decode_amd as gr
    L = gr.lib()
    assert L.gr_abi_version() == 10
    assert L.gr_status_str(-6) == b"max_ctx + 1 tokens exceed the block table's pages"
    assert L.gr_kv_head_bytes(2, 128) == 16 * 128 + 16 * 4 * 2
    assert L.gr_kv_head_bytes(7, 128) == -1
    assert L.gr_stream_read(None, 0, None, None) == 0
    assert L.gr_stream_read(None, 16, None, None) == -1
    # B == 0 is a no-op; NULL pointers, bad K, bad dtype, capacity are rejected
    assert L.gr_q4k_gemm(None, None, None, 0, 16, 256, None, 0, None) == 0
    assert L.gr_q4k_gemm(None, None, None, 1, 16, 256, None, 0, None) == -1
    buf = ctypes.create_string_buffer(4096)
    p = ctypes.addressof(buf) + (-ctypes.addressof(buf) % 256)
    assert L.gr_q4k_gemm(p, p, p, 1, 16, 255, p, 1024, None) == -2
    cfg = gr.layer_cfg(256, 4, 2, 64, 768, 1e-6, 1e4, 0, 0, 5)
    w = gr.LayerWeights(*([p] * 11 + [12] * 7))
    assert L.gr_decode_layer(ctypes.byref(cfg), ctypes.byref(w), p, p, 9, p, p, 9, p, 128, 1, p, 1 << 20, None) == -3
    cfg = gr.layer_cfg(256, 4, 2, 64, 768, 1e-6, 1e4, 0, 0, 0)
    assert L.gr_decode_layer(ctypes.byref(cfg), ctypes.byref(w), p, p, 9, p, p, 8, p, 128, 1, p, 1 << 20, None) == -6
    w2 = gr.LayerWeights(*([p] * 11 + [12] * 6 + [11]))  # Q3_K: not a supported row format
    assert L.gr_decode_layer(ctypes.byref(cfg), ctypes.byref(w2), p, p, 9, p, p, 9, p, 128, 1, p, 1 << 20, None) == -3
    meta = gr.attn_meta(4, 2, 96, 1, 9, 9, 128)
    assert L.gr_paged_decode_attn(p, p, p, p, p, p, 1, ctypes.byref(meta), p, 4096, None) == -2
    meta = gr.attn_meta(4, 2, 64, 1, 9, 8, 129)
    assert L.gr_paged_decode_attn(p, p, p, p, p, p, 1, ctypes.byref(meta), p, 4096, None) == -6
    # the allocation-free variant: the same checks, and a call needing more than its
    # fixed scratch is refused before the device is touched
    assert L.gr_paged_decode_attn_noalloc(p, p, p, p, p, p, 1, ctypes.byref(meta), None) == -6
    assert L.gr_paged_decode_attn_noalloc(None, p, p, p, p, p, 0, ctypes.byref(meta), None) == -6
    meta = gr.attn_meta(64, 8, 128, 1, 1 << 20, 2048, 32768)
    assert L.gr_paged_decode_attn_workspace_size(ctypes.byref(meta), 512) > 16 << 20
    assert L.gr_paged_decode_attn_noalloc(p, p, p, p, p, p, 512, ctypes.byref(meta), None) == -5
    assert L.gr_paged_decode_attn_noalloc(None, p, p, p, p, p, 512, ctypes.byref(meta), None) == -1


def test_gemm_launch_shape_names_the_kernel():
    """The launch-shape query picks the kernel the entry points launch (host-only call)."""
    import continuous_quantized_decode_amd as gr
    q4, q6 = 12, 14
    # Llama-3-8B shapes at B = 8: the output head and the gate/up pairs run the tile loop
    head = gr.gr_gemm_launch_shape(q6, 128256, 4096, 8, gr.GEMM_EPI_STORE)
    assert head["tile_loop"] and head["nt"] == 1 and head["kernel"] == "gemm_tl_kernel<14, 1,"
    gu = gr.gr_gemm_launch_shape(q4, 14336, 4096, 8, gr.GEMM_EPI_SWIGLU)  # whole tiles, a wave per 256 of K
    assert gu["tile_loop"] and gu["whole_tile"] and gu["nt"] == 2 and gu["block_threads"] == 16 * 64
    assert gu["kernel"] == "gemm_tlw_kernel<2>" and gu["grid_threads"] == 256 * 16 * 64
    qkv = gr.gr_gemm_launch_shape(q4, 6144, 4096, 8, gr.GEMM_EPI_STORE)  # Q4_K store from 256 tiles: whole tiles too
    assert qkv["whole_tile"] and qkv["nt"] == 1 and qkv["kernel"] == "gemm_tlw_kernel<0>"
    # residual updates and small matrices keep the split-K kernel
    down = gr.gr_gemm_launch_shape(q6, 4096, 14336, 8, gr.GEMM_EPI_RESIDUAL)  # K-chunk staging: 4 stages of 14
    assert down["k_chunks"] and down["kernel"] == "gemm_kcw_kernel" and down["block_threads"] == 14 * 64
    assert gr.gr_gemm_launch_shape(q6, 1024, 3072, 8, gr.GEMM_EPI_RESIDUAL)["kernel"].startswith("gemm_kernel<14, 1, 1,")
    # a Q4_K residual update from 256 tiles at one batch tile (Wo): whole tiles; at 9 rows: split-K
    assert gr.gr_gemm_launch_shape(q4, 8200, 4096, 8, gr.GEMM_EPI_RESIDUAL)["kernel"] == "gemm_tlw_kernel<1>"
    assert not gr.gr_gemm_launch_shape(q4, 8200, 4096, 9, gr.GEMM_EPI_RESIDUAL)["tile_loop"]
    assert gr.gr_gemm_launch_shape(q4, 8200, 4096, 8, gr.GEMM_EPI_STORE)["tile_loop"]
    # the tile loop's epilogue needs two waves (K of three super-blocks or more)
    assert not gr.gr_gemm_launch_shape(q4, 16384, 512, 8, gr.GEMM_EPI_STORE)["tile_loop"]
    assert gr.gr_gemm_launch_shape(q4, 16384, 768, 8, gr.GEMM_EPI_STORE)["tile_loop"]
    # more than one batch tile, or K above 16 super-blocks: split-K
    # up to 16 rows (two activation tiles) with K of seven super-blocks or more: the tile
    # loop with two batch tiles
    two = gr.gr_gemm_launch_shape(q6, 128256, 4096, 9, gr.GEMM_EPI_STORE)
    assert two["tile_loop"] and two["btn"] == 2 and two["kernel"] == "gemm_tl_kernel<14, 1,"
    assert gr.gr_gemm_launch_shape(q4, 14336, 4096, 16, gr.GEMM_EPI_SWIGLU)["tile_loop"]
    assert not gr.gr_gemm_launch_shape(q4, 16384, 1536, 16, gr.GEMM_EPI_STORE)["tile_loop"]
    assert not gr.gr_gemm_launch_shape(q6, 128256, 4096, 17, gr.GEMM_EPI_STORE)["tile_loop"]
    assert not gr.gr_gemm_launch_shape(q6, 128256, 4352, 8, gr.GEMM_EPI_STORE)["tile_loop"]
    # 17 to 32 rows: the Q4_K gate/up pairs on the row-block kernel (K = 4096: two ranges of
    # eight super-blocks, eight waves, 128 workgroups per range), the plain stores not
    rb = gr.gr_gemm_launch_shape(q4, 12288, 4096, 32, gr.GEMM_EPI_SWIGLU)
    assert rb["row_block"] and rb["kernel"] == "gemm_rb_kernel" and rb["block_threads"] == 8 * 64
    assert rb["grid_threads"] == 256 * 8 * 64
    assert gr.gr_gemm_launch_shape(q4, 12288, 4096, 17, gr.GEMM_EPI_SWIGLU)["row_block"]
    assert not gr.gr_gemm_launch_shape(q4, 12288, 4096, 16, gr.GEMM_EPI_SWIGLU)["row_block"]
    assert not gr.gr_gemm_launch_shape(q4, 12288, 4096, 33, gr.GEMM_EPI_SWIGLU)["row_block"]
    assert not gr.gr_gemm_launch_shape(q4, 6144, 4096, 32, gr.GEMM_EPI_STORE)["row_block"]
    assert not gr.gr_gemm_launch_shape(q6, 12288, 4096, 32, gr.GEMM_EPI_SWIGLU)["row_block"]
    L = gr.lib()
    out = [ctypes.c_int() for _ in range(6)]
    assert L.gr_gemm_launch_shape(q4, 64, 256, 1, 3, *[ctypes.byref(o) for o in out]) == -2
    # more than 64 rows: the many-row kernel (512 threads; groups of 16 weight tiles, or of
    # 8 gate/up pairs, times groups of 4 (Q4_K) or 2 (Q6_K) activation tiles of 8 rows)
    mm = gr.gr_gemm_launch_shape(q4, 14336, 4096, 264, gr.GEMM_EPI_SWIGLU)
    assert mm["many_rows"] and not mm["tile_loop"] and mm["kernel"] == "gemm_mm_kernel<12,"
    assert mm["block_threads"] == 512 and mm["grid_threads"] == (36 // 4) * (896 // 8) * 512
    # 96 workgroups for a narrow matrix: K split in 2 ranges (one round of half the work
    # on 192 CUs; then a finishing pass)
    mm6 = gr.gr_gemm_launch_shape(q6, 4096, 14336, 65, gr.GEMM_EPI_RESIDUAL)
    assert mm6["many_rows"] and mm6["btn"] == 2 and mm6["grid_threads"] == (12 // 2) * (256 // 16) * 2 * 512
    # 288 workgroups: two rounds unsplit, five rounds of a quarter split in 4
    assert gr.gr_gemm_launch_shape(q6, 4096, 14336, 264, 1)["grid_threads"] == 18 * 16 * 4 * 512
    # one full round, or more than 8192 columns: no split
    assert gr.gr_gemm_launch_shape(q4, 4096, 4096, 512)["grid_threads"] == (64 // 4) * 16 * 512
    assert gr.gr_gemm_launch_shape(q4, 9000, 1024, 300)["grid_threads"] == (40 // 4) * 36 * 512
    # Q4_K / Q6_K from 33 rows up take the many-row kernel (measured faster at 64 rows,
    # slower at 32); Q5_K / Q8_0 keep the split-K kernel up to 64 rows
    assert gr.gr_gemm_launch_shape(q4, 4096, 4096, 33)["many_rows"]
    assert not gr.gr_gemm_launch_shape(q4, 4096, 4096, 32)["many_rows"]
    assert not gr.gr_gemm_launch_shape(13, 4096, 4096, 64)["many_rows"]
    assert L.gr_gemm_launch_shape(13, 64, 256, 65, 0, *[ctypes.byref(o) for o in out]) == -3  # Q5_K: at most 64 rows
    assert L.gr_gemm_launch_shape(q4, 64, 256, 513, 0, *[ctypes.byref(o) for o in out]) == -2
    p = ctypes.c_void_p(256)
    assert L.gr_q8_0_gemm(p, p, p, 65, 16, 256, p, 1 << 20, None) == -3
    assert L.gr_q4k_gemm(p, p, p, 513, 16, 256, p, 1 << 20, None) == -2


def test_sample_host_checks_without_gpu():
    import continuous_quantized_decode_amd as gr
    L = gr.lib()
    buf = ctypes.create_string_buffer(1 << 16)
    p = ctypes.addressof(buf) + (-ctypes.addressof(buf) % 256)
    big = 1 << 30
    assert L.gr_sample(None, 0, 10, None, None, None, None, 0, None) == 0
    assert L.gr_sample(p, 1, 0, p, p, None, p, big, None) == -2
    assert L.gr_sample(p, 1, (1 << 18) + 1, p, p, None, p, big, None) == -2
    assert L.gr_sample(p, 65536, 10, p, p, None, p, big, None) == -2
    assert L.gr_sample(None, 1, 10, p, p, None, p, big, None) == -1
    assert L.gr_sample(p, 1, 10, p + 4, p, None, p, big, None) == -4
    assert L.gr_sample(p, 1, 10, p, p, p + 4, p, big, None) == -4
    assert L.gr_sample(p, 1, 10, p, p, None, p, 64, None) == -5
    assert L.gr_sample(p, 1, 10, p, p, None, p + 8, big, None) == -5
    assert L.gr_sample_workspace_size(8, 128256) > 8 * 4096 * 12 > 0
    assert L.gr_sample_workspace_size(8, (1 << 18) + 1) == 0


def test_mixed_stack_head_rows_host_checks():
    """gr_mixed_stack's named logit rows are checked on the host: 1 <= n_head_rows <= rows,
    the index array 4-byte aligned (the indices themselves are clamped on the device)."""
    import continuous_quantized_decode_amd as gr
    L = gr.lib()
    buf = ctypes.create_string_buffer(8192)
    p = ctypes.addressof(buf) + (-ctypes.addressof(buf) % 256)
    cfg = gr.layer_cfg(256, 4, 2, 64, 768, 1e-6, 1e4, 0, 0, 0)
    w = gr.LayerWeights(*([p] * 11 + [12] * 7))
    kp = (ctypes.c_void_p * 1)(p)
    vp = (ctypes.c_void_p * 1)(p)

    def call(head_rows, n_head, rows=4):
        return L.gr_mixed_stack(ctypes.byref(cfg), ctypes.byref(w), 1, kp, vp, 9, p, p, 8, p, p, rows, 100, p, p, 14,
                                1000, head_rows, n_head, p, p, 1 << 24, None)

    assert call(p, 5) == -2      # more named rows than the step has
    assert call(p, 0) == -2
    assert call(p + 2, 2) == -4  # misaligned index array
    assert call(p, 2, rows=513) == -2  # above the 512-row step budget


def test_attn_launch_shape():
    """The decode attention's plan (host-only call): four waves per workgroup, each with
    all of its pages in flight (f32 2, f16 2, q8_0 3 pages); the long-context workload's
    rows take more than 64 workgroups, whose states the last one merges; a context past
    512 workgroups is refused before anything runs, by the decode layer too."""
    import continuous_quantized_decode_amd as gr
    sh = gr.gr_attn_launch_shape(2, 64, 8, 32768 + 1)  # q8_0: 12 pages per workgroup
    assert sh["waves_per_wg"] == 4 and sh["pages_per_wave"] == 3
    assert sh["wg_per_row"] == -(-2049 // 12) > 64
    assert sh["grid_threads"] == 64 * 8 * sh["wg_per_row"] * 256
    llama = gr.gr_attn_launch_shape(1, 8, 8, 3574)  # f16: 8 pages per workgroup
    assert llama["pages_per_wave"] == 2 and llama["wg_per_row"] == 28
    assert gr.gr_attn_launch_shape(1, 8, 8, 16)["wg_per_row"] == 1
    assert gr.gr_attn_launch_shape(0, 1, 1, 16 * 8 + 1)["wg_per_row"] == 2  # f32: 8 pages per workgroup
    assert gr.gr_attn_launch_shape(1, 1, 1, 256 * 16 * 8)["wg_per_row"] == 256
    L = gr.lib()
    v = [ctypes.c_int() for _ in range(3)]
    g = ctypes.c_longlong()
    too_long = 512 * 16 * 8 + 1  # f16: 512 workgroups of 8 pages
    assert L.gr_attn_launch_shape(1, 1, 1, too_long, *[ctypes.byref(i) for i in v], ctypes.byref(g)) == -6
    # the same limit for a decode layer: max_ctx + 1 tokens
    cfg = gr.layer_cfg(256, 4, 2, 64, 768, 1e-6, 1e4, 0, 0, 1)
    buf = ctypes.create_string_buffer(4096)
    p = ctypes.addressof(buf) + (-ctypes.addressof(buf) % 256)
    w = gr.LayerWeights(*([p] * 11 + [12] * 7))
    assert L.gr_decode_layer(ctypes.byref(cfg), ctypes.byref(w), p, p, 9, p, p, 5000, p, too_long - 1, 1, p,
                             1 << 20, None) == -6
