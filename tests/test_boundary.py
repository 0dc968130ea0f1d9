"""The C-ABI library loads, exports every entry point the headers declare, and validates
descriptors on the host (no GPU needed: the device check is replaced by HTGEMM_FAKE_ARCH)."""
import ctypes
import os
import re

import pytest

from hierarchical_tiling_amd import htgemm as H

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = set()
    for hdr in ("htgemm.h", "htlayout.h"):
        text = open(os.path.join(ROOT, "include", hdr)).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s+(\w+)\s*\(", text, re.M):
            names.add(m.group(1))
    return names


def test_every_declared_symbol_is_exported():
    lib = ctypes.CDLL(H.LIB_PATH)
    names = declared_functions()
    assert {"gemm_create", "gemm_run", "gemm_destroy", "ht_layout_compose"} <= names
    for n in sorted(names):
        assert hasattr(lib, n), n
    assert names == set(H.EXPORTED)


@pytest.fixture
def fake_gfx950(monkeypatch):
    monkeypatch.setenv("HTGEMM_FAKE_ARCH", "gfx950")


def desc(**kw):
    base = dict(M=128, N=128, K=64, dtype="bf16", a_strides=(64, 1), b_strides=(1, 64),
                d_strides=(128, 1))
    base.update(kw)
    return H.make_desc(**base)


def status_of(d):
    try:
        h = H.gemm_create(d)
    except H.GemmError as e:
        return e.status
    H.gemm_destroy(h)
    return 0


def test_status_strings():
    assert H.gemm_status_string(0) == "success"
    assert "gfx950" in H.gemm_status_string(5)
    assert H.gemm_status_string(12345) == "unknown status"


def test_valid_descriptor_creates(fake_gfx950):
    assert status_of(desc()) == 0


@pytest.mark.parametrize("mutate,status", [
    (lambda d: setattr(d, "M", -1), 1),
    (lambda d: setattr(d, "split_k", -1), 1),
    (lambda d: setattr(d, "split_k", 65), 1),
    (lambda d: setattr(d, "act", 7), 1),
    (lambda d: setattr(d, "b_type", 1), 2),                      # A bf16 with B fp16
    (lambda d: setattr(d, "d_type", 0), 2),                      # bf16 inputs, fp32 output
    (lambda d: (setattr(d, "has_c", 1), setattr(d, "c_type", 1)), 2),
    (lambda d: (setattr(d, "a_stride_m", 64), setattr(d, "a_stride_k", 2)), 3),  # no unit stride
    (lambda d: setattr(d, "b_stride_n", -64), 3),
    (lambda d: setattr(d, "force_config", 10000), 8),
])
def test_invalid_descriptors(fake_gfx950, mutate, status):
    d = desc()
    mutate(d)
    assert status_of(d) == status


def test_wrong_arch_is_refused(monkeypatch):
    monkeypatch.setenv("HTGEMM_FAKE_ARCH", "gfx942")
    assert status_of(desc()) == 5


def test_destroyed_and_null_handles(fake_gfx950):
    h = H.gemm_create(desc())
    assert H.gemm_workspace_size(h) == 0
    H.gemm_destroy(h)
    assert H.lib().gemm_workspace_size(None, ctypes.byref(ctypes.c_size_t())) == 7
    assert H.lib().gemm_run(None, None, None, None, None, None, 1.0, 0.0, 1.0, 1.0, None, None) == 7
    assert H.lib().gemm_destroy(None) == 0


def test_beta_without_c_and_empty_problem_on_host(fake_gfx950):
    h = H.gemm_create(desc())
    # beta != 0 with a handle that has no C: rejected before any device work
    assert H.lib().gemm_run(h, 16, 16, None, 16, None, 1.0, 0.5, 1.0, 1.0, None, None) == 1
    H.gemm_destroy(h)
    h0 = H.gemm_create(desc(M=0))
    # an empty problem returns success without touching the device
    assert H.lib().gemm_run(h0, None, None, None, None, None, 1.0, 0.0, 1.0, 1.0, None, None) == 0
    H.gemm_destroy(h0)


def test_misaligned_pointer_is_rejected_on_host(fake_gfx950):
    h = H.gemm_create(desc())
    # bf16 pointers must be 2-byte aligned: an odd address is refused before any launch
    assert H.lib().gemm_run(h, 4097, 8192, None, 8192, None, 1.0, 0.0, 1.0, 1.0, None, None) == 4
    H.gemm_destroy(h)


def _info(d):
    h = H.gemm_create(d)
    try:
        return H.gemm_get_info(h)
    finally:
        H.gemm_destroy(h)


def test_tile_table_choices(fake_gfx950):
    names = [H.gemm_config_name(i) for i in range(H.gemm_num_configs())]
    assert len(set(names)) == len(names)
    big = _info(desc(M=8192, N=8192, K=8192, a_strides=(8192, 1), b_strides=(1, 8192), d_strides=(8192, 1)))
    assert (big.bm, big.bn) == (256, 256) and big.name.startswith(b"bf16_ak_bk")
    assert big.grid == 32 * 32
    # ragged fp16 with odd leading dimensions (2-byte aligned rows): this product takes the
    # realigning loader; a large one runs on aligned K-major copies of A and B (K padded to 2056)
    # made in the workspace, with the split ring
    small_rag = _info(H.make_desc(2051, 1533, 1027, "f16", (1027, 1), (1533, 1), (1533, 1)))
    assert b"realign" in small_rag.name and not small_rag.repack
    # fp8 has no realigning loader: copies (row-major B here)
    r8 = _info(H.make_desc(2051, 1533, 1027, "e4m3", (1027, 1), (1533, 1), (1533, 1)))
    assert r8.repack and r8.name.startswith(b"e4m3_ak_bk_")
    d_rag = H.make_desc(4099, 3071, 2053, "f16", (2053, 1), (3071, 1), (3071, 1), c_strides=(3071, 1))
    rag = _info(d_rag)
    assert rag.repack and rag.name.startswith(b"f16_ak_bk_") and rag.config == rag.fallback
    h = H.gemm_create(d_rag)
    try:
        copies = ((4099 * 2056 * 2 + 255) // 256 + (3071 * 2056 * 2 + 255) // 256) * 256
        assert H.gemm_workspace_size(h) == copies      # the ring here needs no split workspace
    finally:
        H.gemm_destroy(h)
    # fp8 has no realigning loader: element loads, or copies where the model predicts them faster
    # (e4m3 301 x 257 x 203: 13.4 us on copies against 14.9 us with element loads)
    rag8 = _info(H.make_desc(301, 257, 203, "e4m3", (203, 1), (1, 203), (257, 1)))
    assert rag8.repack and b"_vec" in rag8.name
    small8 = _info(H.make_desc(120, 257, 203, "e4m3", (203, 1), (1, 203), (257, 1)))
    assert b"narrow" in small8.name and not small8.repack   # below 128 rows: no copies
    # M <= 16 with 16-byte-aligned K-major operands: the streaming (skinny) kernel, one
    # workgroup per 32 output columns
    sk = _info(H.make_desc(16, 16384, 8192, "e4m3", (8192, 1), (1, 8192), (16384, 1)))
    assert b"skinny" in sk.name and sk.bm == 16 and sk.grid == 16384 // 32
    # one more row: back to the tiled kernels
    tall = _info(H.make_desc(17, 16384, 8192, "e4m3", (8192, 1), (1, 8192), (16384, 1)))
    assert b"skinny" not in tall.name
    # a skinny kernel cannot be forced onto M > 16
    names = [H.gemm_config_name(i) for i in range(H.gemm_num_configs())]
    sk_bf16 = names.index("bf16_ak_bk_16x32_w8_skinny")
    assert status_of(desc(M=17, force_config=sk_bf16)) == 8
    assert _info(desc(M=16, force_config=sk_bf16)).config == sk_bf16


def test_forced_config_must_match(fake_gfx950):
    names = [H.gemm_config_name(i) for i in range(H.gemm_num_configs())]
    f16 = names.index("f16_ak_bk_128x128x64_w2x2_m32_vec")
    assert status_of(desc(force_config=f16)) == 8      # bf16 problem, fp16 kernel
    bf = names.index("bf16_ak_bk_128x128x64_w2x2_m32_narrow")
    assert _info(desc(force_config=bf)).config == bf


def test_split_k_plan_and_workspace(fake_gfx950):
    """Split-K ("CUTLASS", Part III: split the K loop when the output has too few tiles): the
    workspace holds one fp32 M x N plane per K slice; slices are whole k-tiles, never empty."""
    # automatic: 1024 x 1024 with K = 65536: 16 tiles of 256 x 256, 16 slices -> 256 workgroups
    h = H.gemm_create(desc(M=1024, N=1024, K=65536, a_strides=(65536, 1), b_strides=(1, 65536),
                           d_strides=(1024, 1)))
    try:
        info = H.gemm_get_info(h)
        assert (info.bm, info.bn) == (256, 256)
        assert info.split_k == 16 and info.grid == 16 * 16
        assert H.gemm_workspace_size(h) == 16 * 1024 * 1024 * 4
        # a split run without a workspace is refused before any launch
        assert H.lib().gemm_run(h, 256, 256, None, 256, None, 1.0, 0.0, 1.0, 1.0, None, None) == 1
    finally:
        H.gemm_destroy(h)
    # 512 x 512 with K = 16384: only 128 x 128 tiles reach 256 workgroups (16 tiles x 16 slices)
    small = _info(desc(M=512, N=512, K=16384, a_strides=(16384, 1), b_strides=(1, 16384),
                       d_strides=(512, 1)))
    assert (small.bm, small.split_k, small.grid) == (128, 16, 256)
    # short K: no split even with few tiles (2048 x 2048 x 2048: 128 x 128 tiles, no split)
    short = _info(desc(M=2048, N=2048, K=2048, a_strides=(2048, 1), b_strides=(1, 2048),
                       d_strides=(2048, 1)))
    assert short.split_k == 1 and short.bm == 128
    # enough tiles: no split and no workspace
    assert _info(desc(M=8192, N=8192, K=65536, a_strides=(65536, 1), b_strides=(1, 65536),
                      d_strides=(8192, 1))).split_k == 1
    # forced: 3 slices of K = 64 * 7 (7 k-tiles of 64) -> 3, 3, 1 k-tiles
    f = _info(desc(K=448, a_strides=(448, 1), b_strides=(1, 448), split_k=3))
    assert f.split_k == 3
    # forced beyond the k-tile count: capped at one slice per k-tile
    assert _info(desc(K=128, a_strides=(128, 1), b_strides=(1, 128), split_k=8)).split_k == 2
    # split_k = 1 never splits
    assert _info(desc(M=1024, N=1024, K=65536, a_strides=(65536, 1), b_strides=(1, 65536),
                      d_strides=(1024, 1), split_k=1)).split_k == 1
    # the streaming skinny kernel takes a forced split along K; the register-staged skinny
    # kernel has none, so forcing both is refused
    names = [H.gemm_config_name(i) for i in range(H.gemm_num_configs())]
    sk = _info(H.make_desc(16, 16384, 8192, "e4m3", (8192, 1), (1, 8192), (16384, 1), split_k=2))
    assert b"skinny_dma" in sk.name and sk.split_k == 2
    assert status_of(desc(M=16, force_config=names.index("bf16_ak_bk_16x32_w8_skinny"), split_k=2)) == 8


def test_scale_vector_and_activation_fields(fake_gfx950):
    """The fused-epilogue fields ("CUTLASS", Part IV Stage 5: per-channel scales and activations
    in the epilogue): flags are 0/1, activations 0..3 (SiLU = 3); a handle with a scale vector
    refuses gemm_run (which cannot pass the vector) before any launch."""
    assert status_of(desc(act="silu")) == 0
    d = desc()
    d.act = 4
    assert status_of(d) == H.GEMM_ERR_INVALID_ARG
    d = desc(row_scale=True)
    d.has_row_scale = 2
    assert status_of(d) == H.GEMM_ERR_INVALID_ARG
    h = H.gemm_create(desc(row_scale=True, col_scale=True))
    try:
        assert H.lib().gemm_run(h, 256, 256, None, 256, None, 1.0, 0.0, 1.0, 1.0, None, None) == 1
        # gemm_run_ex: the vectors must match the handle, and be 4-byte aligned
        run_ex = lambda rs, cs: H.lib().gemm_run_ex(h, H.gemm_args(256, 256, None, 256, None, rs, cs,
                                                                    1.0, 0.0, 1.0, 1.0, None), None)
        assert run_ex(None, 1024) == H.GEMM_ERR_INVALID_ARG
        assert run_ex(1024, None) == H.GEMM_ERR_INVALID_ARG
        assert run_ex(1026, 1024) == H.GEMM_ERR_MISALIGNED
    finally:
        H.gemm_destroy(h)


def test_batch_fields(fake_gfx950):
    """The batch mode (the problem shape's L, "CUTLASS, CuTe, and CUDA Tile", "Assembling a
    CUTLASS kernel"): grid z holds the problems, distinct problems need distinct D, no split-K,
    and the 16-byte kernels only when every problem's A and B stay 16-byte aligned."""
    L = 5
    base = dict(M=512, N=512, K=4096, a_strides=(4096, 1), b_strides=(1, 4096), d_strides=(512, 1))
    ok = _info(desc(batch=L, batch_strides=(512 * 4096, 512 * 4096, 0, 512 * 512), **base))
    assert ok.split_k == 1 and ok.grid == L * (512 // ok.bm) * (512 // ok.bn)
    assert b"_vec" in ok.name or b"_ring" in ok.name or b"_dma" in ok.name
    # 512 x 512 x 65536 alone splits K (16 tiles, 1024 k-tiles); as a batch it never does
    assert _info(desc(batch=L, batch_strides=(0, 0, 0, 512 * 512), **dict(base, K=65536,
                      a_strides=(65536, 1), b_strides=(1, 65536)))).split_k == 1
    # a shared B (stride 0) is allowed; a shared D is not
    assert status_of(desc(batch=L, batch_strides=(512 * 4096, 0, 0, 512 * 512), **base)) == 0
    assert status_of(desc(batch=L, batch_strides=(512 * 4096, 0, 0, 0), **base)) == H.GEMM_ERR_INVALID_ARG
    # negative strides, out-of-range batch, forced split with a batch
    assert status_of(desc(batch=L, batch_strides=(-1, 0, 0, 512 * 512), **base)) == H.GEMM_ERR_LAYOUT
    assert status_of(desc(batch=65536, batch_strides=(0, 0, 0, 512 * 512), **base)) == H.GEMM_ERR_INVALID_ARG
    assert status_of(desc(batch=-1, **base)) == H.GEMM_ERR_INVALID_ARG
    assert status_of(desc(batch=L, split_k=2, batch_strides=(0, 0, 0, 512 * 512), **base)) == H.GEMM_ERR_INVALID_ARG
    # an A stride off the 16-byte grid (odd element count): only the element-wise loaders
    odd = _info(desc(batch=2, batch_strides=(512 * 4096 + 1, 0, 0, 512 * 512), **base))
    assert b"_vec" not in odd.name and b"_ring" not in odd.name and b"_dma" not in odd.name
    # batch 0 and 1 are one problem
    assert _info(desc(batch=0, **base)).grid == _info(desc(batch=1, **base)).grid


def test_grouped_ragged_m_fields(fake_gfx950):
    """Grouped GEMM with ragged M (mixture-of-experts, "CUTLASS", Part V): A K-major, no split,
    no skinny kernel, a grid sized for any split of M into the groups, and each run entry point
    accepts only its own kind of handle (checked before any launch)."""
    G = 8
    base = dict(M=1000, N=512, K=256, a_strides=(256, 1), b_strides=(1, 256), d_strides=(512, 1),
                batch=G, batch_strides=(0, 256 * 512, 0, 0), ragged_m=True)
    info = _info(desc(**base))
    assert info.split_k == 1 and info.grid == (-(-1000 // info.bm) + G) * (512 // info.bn)
    assert status_of(desc(**dict(base, a_strides=(1, 1000)))) == H.GEMM_ERR_LAYOUT
    assert status_of(desc(**dict(base, split_k=2))) == H.GEMM_ERR_INVALID_ARG
    d = desc(**base)
    d.ragged_m = 2
    assert status_of(d) == H.GEMM_ERR_INVALID_ARG
    # the batch field counts the groups (offsets holds batch + 1 values): at least one group
    for groups in (0, -1):
        assert status_of(desc(**dict(base, batch=groups))) == H.GEMM_ERR_INVALID_ARG
    assert _info(desc(**dict(base, batch=1))).split_k == 1
    small = _info(H.make_desc(16, 16384, 8192, "e4m3", (8192, 1), (1, 8192), (16384, 1), batch=4,
                              batch_strides=(0, 16384 * 8192, 0, 0), ragged_m=True))
    assert b"skinny" not in small.name
    args = H.gemm_args(256, 256, None, 256, None, None, None, 1.0, 0.0, 1.0, 1.0, None)
    h = H.gemm_create(desc(**base))
    try:
        assert H.lib().gemm_run(h, 256, 256, None, 256, None, 1.0, 0.0, 1.0, 1.0, None, None) == 1
        assert H.lib().gemm_run_ex(h, ctypes.byref(args), None) == 1
        assert H.lib().gemm_run_grouped(h, ctypes.byref(args), None, None) == 1
        assert H.lib().gemm_run_grouped(h, ctypes.byref(args), 1026, None) == H.GEMM_ERR_MISALIGNED
    finally:
        H.gemm_destroy(h)
    h = H.gemm_create(desc())
    try:   # a plain handle refuses the grouped entry point
        assert H.lib().gemm_run_grouped(h, ctypes.byref(args), 1024, None) == 1
    finally:
        H.gemm_destroy(h)


def test_grouped_problems_fields(fake_gfx950):
    """Grouped GEMM of independent problems ("CUTLASS", Part III: many problems of irregular
    shapes in one launch): the descriptor fixes types, layouts and epilogue; the run's host
    checks refuse bad problems before anything reaches the device."""
    G = 5
    base = dict(M=512, N=512, K=256, a_strides=(256, 1), b_strides=(1, 256), d_strides=(512, 1),
                batch=G, grouped=True)
    info = _info(desc(**base))
    assert info.split_k == 1 and b"skinny" not in info.name
    h = H.gemm_create(desc(**base))
    try:
        # the problem table (112 bytes a problem, padded to 256) and G + 1 first tiles
        assert H.gemm_workspace_size(h) == (112 * G + 255) // 256 * 256 + (G + 1) * 8
        lib = H.lib()
        args = H.gemm_args(None, None, None, None, None, None, None, 1.0, 0.0, 1.0, 1.0, 4096)
        good = dict(M=64, N=64, K=64, A=256, B=256, D=256, lda=64, ldb=64, ldd=64)

        def rc(problems, a=args, count=None, handle=h):
            arr = (H.gemm_problem * max(len(problems), 1))()
            for i, q in enumerate(problems):
                arr[i] = H.gemm_problem(q["M"], q["N"], q["K"], q.get("A"), q.get("B"),
                                        q.get("C"), q.get("D"), q.get("bias"), q.get("lda", 0),
                                        q.get("ldb", 0), q.get("ldc", 0), q.get("ldd", 0))
            n = len(problems) if count is None else count
            return lib.gemm_run_problems(handle, arr, n, ctypes.byref(a), None)

        # nothing to do: no problems, or only empty ones (no device call is made)
        assert rc([]) == 0
        assert rc([dict(good, M=0), dict(good, N=0, D=None)]) == 0
        assert rc([good] * (G + 1)) == H.GEMM_ERR_INVALID_ARG           # more than batch
        assert rc([good], count=-1) == H.GEMM_ERR_INVALID_ARG
        assert rc([dict(good, M=-1)]) == H.GEMM_ERR_INVALID_ARG
        assert rc([dict(good, ldb=-64)]) == H.GEMM_ERR_LAYOUT
        assert rc([dict(good, D=None)]) == H.GEMM_ERR_INVALID_ARG
        assert rc([dict(good, A=None)]) == H.GEMM_ERR_INVALID_ARG
        assert rc([good, dict(good, D=257)]) == H.GEMM_ERR_MISALIGNED   # odd address, 2-byte D
        # per-operand pointers belong to the problems, not to the arguments
        for field in ("A", "B", "D"):
            bad = H.gemm_args(None, None, None, None, None, None, None, 1.0, 0.0, 1.0, 1.0, 4096)
            setattr(bad, field, 256)
            assert rc([good], a=bad) == H.GEMM_ERR_INVALID_ARG
        beta = H.gemm_args(None, None, None, None, None, None, None, 1.0, 0.5, 1.0, 1.0, 4096)
        assert rc([good], a=beta) == H.GEMM_ERR_INVALID_ARG             # beta without C
        # the other entry points refuse a grouped handle, and this one any other handle
        assert lib.gemm_run(h, 256, 256, None, 256, None, 1.0, 0.0, 1.0, 1.0, None, None) == 1
        plain_args = H.gemm_args(256, 256, None, 256, None, None, None, 1.0, 0.0, 1.0, 1.0, None)
        assert lib.gemm_run_ex(h, ctypes.byref(plain_args), None) == 1
        assert lib.gemm_run_noalloc(h, ctypes.byref(plain_args), None) == 1
        plain = H.gemm_create(desc())
        try:
            assert rc([good], handle=plain) == H.GEMM_ERR_INVALID_ARG
        finally:
            H.gemm_destroy(plain)
    finally:
        H.gemm_destroy(h)
    for bad, status in ((dict(batch=0), H.GEMM_ERR_INVALID_ARG),
                        (dict(split_k=2), H.GEMM_ERR_INVALID_ARG),
                        (dict(ragged_m=True), H.GEMM_ERR_INVALID_ARG),
                        (dict(row_scale=True), H.GEMM_ERR_INVALID_ARG),
                        (dict(d_strides=(1024, 2)), H.GEMM_ERR_LAYOUT)):
        assert status_of(desc(**dict(base, **bad))) == status, bad
    d = desc(**base)
    d.grouped = 3
    assert status_of(d) == H.GEMM_ERR_INVALID_ARG
    # a column-major D is accepted (ldd then replaces the column stride)
    assert status_of(desc(**dict(base, d_strides=(1, 512)))) == 0


def test_stream_k_plan(fake_gfx950):
    """Stream-K ("CUTLASS", Part IV Stage 2): the tiles of a last partial round of a
    one-workgroup-per-CU kernel run as 256 persistent workgroups; the library plans it where it
    was measured to pay (a last round at most half full, at least 64 k-tiles) in place of the
    split tail, for the entries that have a Stream-K form."""
    ring = [H.gemm_config_name(j) for j in range(H.gemm_num_configs())].index(
        "bf16_ak_bk_256x256x64_w2x4_m16_ring")

    def info(M, N, K, **kw):
        g = H.Gemm(H.make_desc(M, N, K, "bf16", (K, 1), (1, K), (N, 1), **kw))
        return g.info, g.workspace_bytes
    ws_sk = 2 * 256 * 256 * 256 * 4
    # the ring that has a Stream-K form, with the library deciding the decomposition
    i, ws = info(4352, 4352, 4096, force_config=ring)   # 289 tiles: 33 in the last round
    assert (i.sk_tiles, i.sk_wgs) == (33, 256) and ws == ws_sk
    assert (i.tail_tiles, i.tail_split) == (0, 1)
    assert info(6144, 6144, 8192, force_config=ring)[0].sk_tiles == 64
    for shape in ((8192, 8192, 8192),       # whole rounds
                  (5120, 5120, 8192),       # 144 left: more than half a round
                  (3840, 3840, 8192),       # one round
                  (6144, 6144, 2048)):      # 32 k-tiles: too shallow
        i, _ = info(*shape, force_config=ring)
        assert i.sk_tiles == 0, shape
    # no Stream-K when asked for none (the split tail then), or with a fixed split
    i, _ = info(4352, 4352, 4096, force_config=ring, decomposition=1)
    assert i.sk_tiles == 0 and i.tail_split > 1
    assert info(4352, 4352, 4096, force_config=ring, split_k=1)[0].sk_tiles == 0
    # the automatic choice compares the plans: here an entry with the split tail (the ping-pong
    # kernel, which has no Stream-K form) is predicted (and was measured) faster than the ring
    # with Stream-K
    i, _ = info(4352, 4352, 4096)
    assert i.name.decode().endswith("_pp") and i.sk_tiles == 0 and i.tail_split > 1
    # forced: every tile when they fit in one round, else the last partial round (the last
    # round with whole rounds only)
    assert info(1000, 1300, 64, force_config=ring, decomposition=2)[0].sk_tiles == 24
    assert info(5120, 5120, 8192, force_config=ring, decomposition=2)[0].sk_tiles == 144
    i, ws = info(8192, 8192, 8192, force_config=ring, decomposition=2)
    assert i.sk_tiles == 256 and ws == ws_sk
    # a kernel without a Stream-K form (an fp32 tile kernel, the fp8 ring and ping-pong kernels)
    # runs data-parallel, or with the split tail
    g = H.Gemm(H.make_desc(512, 512, 512, "f32", (512, 1), (1, 512), (512, 1), decomposition=2))
    assert g.info.sk_tiles == 0 and g.workspace_bytes == 0
    g = H.Gemm(H.make_desc(4352, 4352, 8192, "e4m3", (8192, 1), (1, 8192), (4352, 1)))
    assert g.info.name.decode().endswith(("_ring", "_pp")) and g.info.sk_tiles == 0
    assert g.info.tail_split > 1
    for bad in (dict(decomposition=3), dict(decomposition=-1), dict(decomposition=2, split_k=2),
                dict(decomposition=2, batch=2, batch_strides=(8192 * 8192, 8192 * 8192, 0,
                                                              8192 * 8192))):
        assert status_of(desc(**bad)) == H.GEMM_ERR_INVALID_ARG, bad


def test_row_sumsq_fields(fake_gfx950):
    """The fused row reduction ("CUTLASS", Part IV Stage 5: a reduction for the next layer's
    norm): one problem, no split, no skinny kernel, a workspace of one fp32 partial per tile
    column and row, and gemm_run_ex only (checked before any launch)."""
    i = _info(desc(M=16, N=1040, K=512, a_strides=(512, 1), b_strides=(1, 512),
                   d_strides=(1040, 1), row_sumsq=True))
    assert b"skinny" not in i.name and i.split_k == 1
    h = H.gemm_create(desc(M=300, N=600, K=256, a_strides=(256, 1), b_strides=(1, 256),
                           d_strides=(600, 1), row_sumsq=True))
    try:
        info = H.gemm_get_info(h)
        assert H.gemm_workspace_size(h) >= -(-600 // info.bn) * 300 * 4
        assert H.lib().gemm_run(h, 256, 256, None, 256, None, 1.0, 0.0, 1.0, 1.0, 1024, None) == 1
        run_ex = lambda ws, rsq: H.lib().gemm_run_ex(h, H.gemm_args(256, 256, None, 256, None, None,
                                                                    None, 1.0, 0.0, 1.0, 1.0, ws,
                                                                    rsq), None)
        assert run_ex(1024, None) == H.GEMM_ERR_INVALID_ARG      # the handle expects the vector
        assert run_ex(None, 1024) == H.GEMM_ERR_INVALID_ARG      # the workspace is required
        assert run_ex(1024, 1026) == H.GEMM_ERR_MISALIGNED
    finally:
        H.gemm_destroy(h)
    for bad in (dict(split_k=2), dict(batch=2, batch_strides=(0, 0, 0, 128 * 128)),
                dict(batch=2, batch_strides=(0, 0, 0, 0), ragged_m=True)):
        assert status_of(desc(row_sumsq=True, **bad)) == H.GEMM_ERR_INVALID_ARG


def test_col_sum_fields(fake_gfx950):
    """Column sums of D: the same conditions as the row reduction, and a workspace holding the
    row partials followed by one fp32 partial per (tile row, row group, column)."""
    base = dict(M=300, N=600, K=256, a_strides=(256, 1), b_strides=(1, 256), d_strides=(600, 1))
    h = H.gemm_create(desc(col_sum=True, **base))
    try:
        info = H.gemm_get_info(h)
        groups = max(info.waves // (info.bn // 64), 1)
        assert H.gemm_workspace_size(h) >= -(-300 // info.bm) * groups * 600 * 4
        args = H.gemm_args(256, 256, None, 256, None, None, None, 1.0, 0.0, 1.0, 1.0, 1024, None, None)
        assert H.lib().gemm_run_ex(h, ctypes.byref(args), None) == H.GEMM_ERR_INVALID_ARG
    finally:
        H.gemm_destroy(h)
    only_rows = H.gemm_create(desc(row_sumsq=True, **base))
    both = H.gemm_create(desc(col_sum=True, row_sumsq=True, **base))
    try:
        assert H.gemm_workspace_size(both) > H.gemm_workspace_size(only_rows)
    finally:
        H.gemm_destroy(both)
        H.gemm_destroy(only_rows)
    assert status_of(desc(col_sum=True, split_k=3, **base)) == H.GEMM_ERR_INVALID_ARG
    d = desc(**base)
    d.has_col_sum = 2
    assert status_of(d) == H.GEMM_ERR_INVALID_ARG


# Kernel choice for mid-size and large bf16 products (A row-major, B column-major), from the cost
# model (the fitting entry with the least predicted time).  Each expectation below was measured on
# MI355X against the rule-based choice the model replaced (microseconds, one box):
#   3072^3         the ping-pong kernel 63-68; 256 x 256 DMA entry 67, the ring 70
#   2816^2 x 4096  the ping-pong kernel in 2 slices 75; 128 x 256 DMA tiles 74, 256 x 128 tiles
#                  unsplit 75 (within the model's tie margin)
#   1536^2 x 8192  the ping-pong kernel in 6 slices 56 (the best entry measured)
#   2048^2 x 4096  128 x 128 tiles unsplit 50-53; 4 ring slices of 16 k-tiles 55
#   2048 x 4096 x 2048  half-size (128 x 256 or 256 x 128) tiles 42-44, the ring 51
#   4352^2 x 4096  the ping-pong kernel with the split tail 155-162; a ring with the split tail
#                  167-169; the ring with Stream-K 184
@pytest.mark.parametrize("shape,tile,split,tail,sk", [
    ((3072, 3072, 3072), (256, 256), 1, (0, 1), 0),
    ((3328, 3328, 4096), (256, 256), 1, (0, 1), 0),
    ((2816, 2816, 4096), (256, 256), 2, (0, 1), 0),
    ((1536, 1536, 8192), (256, 256), 6, (0, 1), 0),
    ((2048, 2048, 4096), (128, 128), 1, (0, 1), 0),
    ((2048, 4096, 2048), (256, 128), 1, (0, 1), 0),
    ((2048, 2048, 2048), (128, 128), 1, (0, 1), 0),
    ((512, 512, 16384), (128, 128), 16, (0, 1), 0),
    ((8192, 8192, 8192), (256, 256), 1, (0, 1), 0),
    ((4352, 4352, 4096), (256, 256), 1, (33, 7), 0),
])
def test_kernel_choice_by_rounds(fake_gfx950, shape, tile, split, tail, sk):
    M, N, K = shape
    info = _info(desc(M=M, N=N, K=K, a_strides=(K, 1), b_strides=(1, K), d_strides=(N, 1)))
    name = info.name.decode()
    assert (info.bm * info.bn == tile[0] * tile[1] and info.bm >= 128), name
    assert (info.split_k, info.tail_tiles, info.tail_split, info.sk_tiles) == (split,) + tail + (sk,), name
    assert info.predicted_us > 0


def test_headline_product_runs_on_the_ping_pong_kernel(fake_gfx950):
    """bf16 8192^3 (A row-major, B column- or row-major): the ping-pong kernel (16 x 16 atoms),
    whole rounds, no split (measured 0.78 and 0.83 ms against 0.85 and 0.95 ms on the split
    ring)."""
    for b in ((1, 8192), (8192, 1)):
        info = _info(desc(M=8192, N=8192, K=8192, a_strides=(8192, 1), b_strides=b,
                          d_strides=(8192, 1), has_bias=True, act="gelu"))
        assert info.name.decode().endswith("_w2x4_m16_pp"), info.name
        assert (info.split_k, info.sk_tiles, info.tail_tiles, info.repack) == (1, 0, 0, 0)


@pytest.mark.parametrize("dtype,shape,orders,kernel,repack", [
    ("bf16", (1024, 1024, 1024), ("row", "col"), "_64x64x64_w2x2_m16_vec", 0),     # 256 small tiles
    ("e4m3", (1024, 1024, 1024), ("row", "col"), "_64x64x128_w2x2_m16_vec", 0),
    # 144 of 128x128: predicted 15.5 us against 15.1 us on 64x64, a tie that goes to the entry
    # with the lower sustained cost (measured 16.0-16.8 against 15.1 us)
    ("bf16", (1536, 1536, 1024), ("row", "col"), "_128x128x64_w2x2_m32_vec", 0),
    ("bf16", (2048, 2048, 2048), ("row", "col"), "_128x128x64_w2x2_m32_vec", 0),
    # odd leading dimensions: realigned loaders, or aligned K-major copies where the model
    # predicts them faster (f16 1001^3-ish: 16.7 us on copies against 23-25 us realigned)
    ("f16", (1001, 999, 1003), ("row", "row"), "_64x64x64_w2x2_m16_vec", 1),
    ("f16", (2051, 1533, 1027), ("row", "row"), "_128x128x64_w2x2_m32_realign", 0),
    ("f16", (4099, 3071, 2053), ("row", "row"), "_ak_bk_256x256x64_w2x4_m16_pp", 1),
])
def test_kernel_choice_small_and_realigned(fake_gfx950, dtype, shape, orders, kernel, repack):
    M, N, K = shape
    a = (K, 1) if orders[0] == "row" else (1, M)
    b = (N, 1) if orders[1] == "row" else (1, K)
    info = _info(desc(M=M, N=N, K=K, dtype=dtype, a_strides=a, b_strides=b, d_strides=(N, 1)))
    assert info.name.decode().endswith(kernel), info.name.decode()
    assert info.repack == repack


@pytest.mark.parametrize("L,shape,tile", [
    (16, (1024, 1024, 512), (256, 256)),          # 16 tiles x 16 problems fill one round
    (64, (256, 256, 1024), (128, 128)),
    (1, (1024, 1024, 1024), (64, 64)),
])
def test_kernel_choice_counts_batch_problems(fake_gfx950, L, shape, tile):
    M, N, K = shape
    d = desc(M=M, N=N, K=K, a_strides=(K, 1), b_strides=(1, K), d_strides=(N, 1), batch=L,
             batch_strides=(M * K, N * K, 0, M * N))
    info = _info(d)
    assert (info.bm, info.bn) == tile, info.name


def test_noalloc_scratch_limit_and_arguments(fake_gfx950):
    """gemm_run_noalloc refuses, before touching the device, a handle whose workspace exceeds the
    static scratch, a caller workspace, and a grouped handle."""
    big = H.gemm_create(H.make_desc(2048, 2048, 65536, "bf16", (65536, 1), (1, 65536), (2048, 1),
                                    split_k=8))
    try:
        assert H.gemm_workspace_size(big) > H.GEMM_NOALLOC_SCRATCH_BYTES
        args = H.gemm_args(256, 256, None, 256, None, None, None, 1.0, 0.0, 1.0, 1.0, None)
        assert H.lib().gemm_run_noalloc(big, ctypes.byref(args), None) == H.GEMM_ERR_SCRATCH_LIMIT
        args.workspace = 256
        assert H.lib().gemm_run_noalloc(big, ctypes.byref(args), None) == H.GEMM_ERR_INVALID_ARG
    finally:
        H.gemm_destroy(big)
    assert H.lib().gemm_run_noalloc(None, None, None) == 7   # GEMM_ERR_BAD_HANDLE
    assert H.gemm_status_string(H.GEMM_ERR_SCRATCH_LIMIT).startswith("the problem needs more")


def test_kernel_choice_for_the_misjudged_fp8_product(fake_gfx950):
    """e4m3 3001 x 2999 x 2049 with odd leading dimensions: element-wise loads took 533 us
    (64 x 64) and 628 us (128 x 128) on MI355X; the library copies A and B to aligned K-major
    buffers and runs a 256 x 256 kernel on them (measured with the copies: 59.4 us on the split
    ring, 61.2-62.5 us on the ping-pong kernel; the model puts the two within its tie band)."""
    info = _info(H.make_desc(3001, 2999, 2049, "e4m3", (2049, 1), (1, 2049), (2999, 1)))
    assert info.repack == 1 and info.name in (b"e4m3_ak_bk_256x256x128_w2x4_m32_ring",
                                              b"e4m3_ak_bk_256x256x128_w2x4_m16_pp")


def test_clock_record_arguments(fake_gfx950):
    # host-side checks only: no device memory is touched
    import ctypes
    h = H.gemm_create(desc(M=512, N=512, K=256))
    try:
        L = H.lib()
        assert L.gemm_set_clock_record(None, None, 0) == 7  # GEMM_ERR_BAD_HANDLE
        assert L.gemm_set_clock_record(h, ctypes.c_void_p(0x1000), -1) == H.GEMM_ERR_INVALID_ARG
        assert L.gemm_set_clock_record(h, ctypes.c_void_p(0x1004), 4) == H.GEMM_ERR_INVALID_ARG
        assert L.gemm_set_clock_record(h, ctypes.c_void_p(0x1000), 4) == 0
        assert L.gemm_set_clock_record(h, None, 0) == 0
    finally:
        H.gemm_destroy(h)


@pytest.mark.parametrize("shape,dtype,split", [
    # few column blocks and long K: K slices (measured 31.8 -> 11.7, 33.1 -> 12.4,
    # 11.0 -> 10.1, 60.5 -> 33.2 us)
    ((16, 16, 32768), "bf16", 8), ((16, 256, 32768), "bf16", 8), ((16, 1024, 8192), "bf16", 4),
    ((16, 2048, 32768), "bf16", 8),
    # enough column blocks or short K: no split (measured faster unsplit)
    ((16, 4096, 4096), "bf16", 1), ((16, 8192, 8192), "bf16", 1), ((8, 4096, 4096), "e4m3", 1),
    ((16, 16384, 8192), "e4m3", 1),
])
def test_skinny_split_choice(fake_gfx950, shape, dtype, split):
    M, N, K = shape
    info = _info(H.make_desc(M, N, K, dtype, (K, 1), (1, K), (N, 1)))
    assert b"skinny_dma" in info.name and info.split_k == split, (info.name, info.split_k)
