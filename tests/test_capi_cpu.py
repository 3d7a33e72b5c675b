"""Host side of the C ABI, on the CPU: exports, packer parity with the oracle,
error codes and the shape contract.  No GPU call is made here."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import verify_nvfp4_w4a16_amd as nv
import workload

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "nvfp4_w4a16.h")


def _declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|const char\*)\s+((?:nvfp4|fp8)_\w+)\s*\(", text, re.M)))


PAGES = ('"10 Kernels"', '"CUDA Kernel Engineering"', '"Module ops"')


def _declaration_comments():
    """{function: the comment block right above its declaration}."""
    text = open(HEADER).read()
    out = {}
    for m in re.finditer(r"/\*(?:(?!\*/).)*\*/\s*(?:(?:int|const char\*)\s+)((?:nvfp4|fp8)_\w+)\s*\(", text, re.S):
        out[m.group(1)] = m.group(0)
    return out


def test_every_declaration_cites_a_passage():
    # Each entry point's comment names the page (and section or entry) that
    # defines what it does, or, for the entry point that allocates nothing,
    # the callers it is for.
    comments = _declaration_comments()
    assert set(comments) == set(_declared_functions())
    for name, block in comments.items():
        if name == "nvfp4_strerror":
            continue                      # static text of the status codes
        cited = any(p in block for p in PAGES) or "cannot allocate" in block
        assert cited, f"{name}: no passage cited in its declaration comment"


def test_library_exports_every_declared_function():
    declared = _declared_functions()
    assert set(declared) == set(nv.EXPORTED)
    lib = ctypes.CDLL(nv.LIB_PATH)
    for name in declared:
        assert hasattr(lib, name), name


def test_header_constants_match_binding():
    text = open(HEADER).read()
    def enum(name):
        return int(re.search(rf"\b{name}\s*=\s*(-?\d+)", text).group(1))
    assert enum("NVFP4_OK") == nv.OK
    for py, c in [(nv.ERR_NULL, "NVFP4_ERR_NULL"), (nv.ERR_SHAPE, "NVFP4_ERR_SHAPE"),
                  (nv.ERR_ALIGN, "NVFP4_ERR_ALIGN"), (nv.ERR_DTYPE, "NVFP4_ERR_DTYPE"),
                  (nv.ERR_NONFINITE, "NVFP4_ERR_NONFINITE"), (nv.ERR_BADSCALE, "NVFP4_ERR_BADSCALE"),
                  (nv.ERR_HIP, "NVFP4_ERR_HIP"), (nv.ERR_DEVICE, "NVFP4_ERR_DEVICE"),
                  (nv.ERR_TILEFILE, "NVFP4_ERR_TILEFILE"), (nv.ERR_BUFFER, "NVFP4_ERR_BUFFER"),
                  (nv.ERR_TILE, "NVFP4_ERR_TILE"), (nv.ERR_SCRATCH, "NVFP4_ERR_SCRATCH"),
                  (nv.ERR_LIBRARY, "NVFP4_ERR_LIBRARY"),
                  (nv.OUT_BF16, "NVFP4_OUT_BF16"), (nv.OUT_F32, "NVFP4_OUT_F32")]:
        assert enum(c) == py, c
    assert int(re.search(r"#define NVFP4_MAX_M (\d+)", text).group(1)) == nv.MAX_M
    assert int(re.search(r"#define NVFP4_K_MULTIPLE (\d+)", text).group(1)) == nv.K_MULTIPLE


def _assert_pack_matches_oracle(w):
    p, s, t = nv.pack(w)
    p2, s2, t2 = oracle.quantize_ref(w)
    assert np.float32(t) == np.float32(t2)
    assert np.array_equal(s, s2)
    assert np.array_equal(p, p2)


@pytest.mark.parametrize("n,k,seed", [(1, 16, 1), (3, 32, 2), (17, 256, 3), (64, 1024, 4)])
def test_pack_matches_oracle_random(n, k, seed):
    _assert_pack_matches_oracle(workload.weights_f32(n, k, seed))


def test_pack_matches_oracle_multithreaded():
    # Large enough that the packer spreads rows over several threads.
    _assert_pack_matches_oracle(workload.weights_f32(1536, 2048, 5))


def test_pack_matches_oracle_adversarial():
    g = workload.rng(6)
    n, k = 64, 256
    w = (g.standard_normal((n, k)) * np.exp(g.uniform(-30, 10, (n, 1)))).astype(np.float32)
    w[0] = 0.0                                   # zero row
    w[1, :16] = 0.0                              # zero group
    w[2, :16] = 1e-40                            # fp32 subnormals
    w[3] = np.float32(3e38)                      # huge values
    w[4, ::7] = -w[4, ::7]
    # exact ties: values at midpoints of the e2m1 grid relative to the group max 6
    ties = np.array([6, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5, -0.25, -0.75, -1.25, -1.75,
                     -2.5, -3.5, -5, 0.0], np.float32)
    w[5, :16] = ties * np.float32(2.0 ** -3)
    _assert_pack_matches_oracle(w)
    # groups made of one repeated value hit every e4m3 code's neighbourhood
    v = np.exp(g.uniform(np.log(1e-8), np.log(1e3), (n * k // 16,))).astype(np.float32)
    w2 = np.repeat(v, 16).reshape(n, k)
    _assert_pack_matches_oracle(w2)


def test_pack_round_trip_closed_form():
    # Weights that are exactly t * e4m3 * e2m1 come back unchanged.
    g = workload.rng(7)
    n, k = 8, 64
    t = float(np.float32(0.75 * 2.0 ** -9))
    s = g.integers(1, 0x7E, size=(n, k // 16), dtype=np.uint8)
    s[0, 0] = 0x7E
    codes = g.integers(1, 8, size=(n, k), dtype=np.uint8) | (g.integers(0, 2, (n, k), dtype=np.uint8) << 3)
    codes[:, ::16] = 7                             # every group's max |code| is 6
    w = (t * oracle.E4M3[s][:, np.arange(k) // 16] * oracle.E2M1[codes]).astype(np.float32)
    p, s2, t2 = nv.pack(w)
    assert t2 == t and np.array_equal(s2, s)
    assert np.array_equal(p, (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8))


def test_pack_errors():
    with pytest.raises(nv.Nvfp4Error) as e:
        nv.pack(np.full((2, 16), np.nan, np.float32))
    assert e.value.status == nv.ERR_NONFINITE
    with pytest.raises(nv.Nvfp4Error) as e:
        nv.pack(np.full((2, 16), -np.inf, np.float32))
    assert e.value.status == nv.ERR_NONFINITE
    with pytest.raises(nv.Nvfp4Error) as e:
        nv.pack(np.zeros((2, 24), np.float32))
    assert e.value.status == nv.ERR_SHAPE
    with pytest.raises(nv.Nvfp4Error) as e:
        nv.pack(np.zeros((0, 16), np.float32))
    assert e.value.status == nv.ERR_SHAPE
    lib = nv._lib()
    t = ctypes.c_float()
    assert lib.nvfp4_pack(None, 1, 16, None, None, ctypes.byref(t)) == nv.ERR_NULL


def test_check_scales():
    s = np.arange(0x7F, dtype=np.uint8).reshape(127, 1)
    assert nv.check_scales(s) == nv.OK
    for bad in (0x7F, 0xFF, 0x80, 0x81, 0xFE):
        s2 = np.zeros((4, 2), np.uint8)
        s2[3, 1] = bad
        assert nv.check_scales(s2) == nv.ERR_BADSCALE
    assert nv._lib().nvfp4_check_scales(None, 1, 16) == nv.ERR_NULL
    assert nv._lib().nvfp4_check_scales(s.ctypes.data, 1, 8) == nv.ERR_SHAPE


@pytest.mark.parametrize("m,n,k,ok", [
    (0, 1, 256, True), (1, 1, 256, True), (32, 151552, 4096, True), (33, 16, 256, False),
    (-1, 16, 256, False), (1, 0, 256, False), (1, 16, 128, False), (1, 16, 384, False),
    (1, 16, 512, True), (16, 4096, 12288, True), (1, 1 << 28, 256, True), (1, (1 << 28) + 1, 256, False),
    (1, 16, 1 << 20, True), (1, 16, (1 << 20) + 256, False)])
def test_shape_contract(m, n, k, ok):
    assert nv.linear_shape_ok(m, n, k) == ok


def test_linear_validates_before_any_device_call():
    lib = nv._lib()
    buf = (ctypes.c_uint8 * 64)()
    a = ctypes.addressof(buf)
    a16 = (a + 15) & ~15
    # shape errors first, then dtype, then M == 0 (no launch), then pointers, then alignment
    assert lib.nvfp4_linear(a16, a16, a16, 1.0, a16, 33, 16, 256, 0, None) == nv.ERR_SHAPE
    assert lib.nvfp4_linear(a16, a16, a16, 1.0, a16, 1, 16, 100, 0, None) == nv.ERR_SHAPE
    assert lib.nvfp4_linear(a16, a16, a16, 1.0, a16, 1, 16, 256, 7, None) == nv.ERR_DTYPE
    assert lib.nvfp4_linear(None, None, None, 1.0, None, 0, 16, 256, 0, None) == nv.OK
    assert lib.nvfp4_linear(None, a16, a16, 1.0, a16, 1, 16, 256, 0, None) == nv.ERR_NULL
    assert lib.nvfp4_linear(a16, a16, a16, 1.0, None, 1, 16, 256, 1, None) == nv.ERR_NULL
    assert lib.nvfp4_linear(a16 + 2, a16, a16, 1.0, a16, 1, 16, 256, 0, None) == nv.ERR_ALIGN
    assert lib.nvfp4_linear(a16, a16 + 8, a16, 1.0, a16, 1, 16, 256, 0, None) == nv.ERR_ALIGN
    assert lib.nvfp4_linear(a16, a16, a16 + 1, 1.0, a16, 1, 16, 256, 0, None) == nv.ERR_ALIGN
    assert lib.nvfp4_linear(a16, a16, a16, 1.0, a16 + 1, 1, 16, 256, 0, None) == nv.ERR_ALIGN
    assert lib.nvfp4_linear(a16, a16, a16, 1.0, a16 + 2, 1, 16, 256, 1, None) == nv.ERR_ALIGN


def test_tiled_entry_validates_the_tile():
    lib = nv._lib()
    buf = (ctypes.c_uint8 * 64)()
    a16 = (ctypes.addressof(buf) + 15) & ~15
    def call(cols, waves, unroll, k=1024, m=1, split=1, mwaves=0, kernel=nv.KERNEL_AUTO):
        t = nv.Tile(cols, waves, unroll, split, mwaves, kernel)
        return lib.nvfp4_linear_tiled(a16, a16, a16, 1.0, a16, m, 16, k, 0, ctypes.byref(t), None)
    assert call(48, 2, 2) == nv.ERR_TILE
    assert call(16, 3, 2) == nv.ERR_TILE
    assert call(16, 2, 3) == nv.ERR_TILE
    assert call(16, 8, 2) == nv.ERR_TILE             # 1024 / 8 = 128 < 2 * 128
    assert call(16, 16, 1, k=8192) == nv.ERR_TILE    # more than 8 wavefronts
    assert call(16, 4, 2, split=3) == nv.ERR_TILE    # split not a power of two
    assert call(16, 2, 2, split=4) == nv.ERR_TILE    # more groups than segments
    assert call(16, 4, 2, mwaves=2) == nv.ERR_TILE   # many-row workgroups are 4, 6 or 8 wavefronts
    assert call(16, 4, 2, kernel=6) == nv.ERR_TILE   # no such kernel
    assert call(16, 4, 2, kernel=-1) == nv.ERR_TILE
    assert call(16, 2, 2, k=100) == nv.ERR_SHAPE
    assert call(16, 2, 2, m=0) == nv.OK              # M == 0: nothing launched
    assert lib.nvfp4_linear_tiled(a16, a16, a16, 1.0, a16, 1, 16, 1024, 0, None, None) == nv.ERR_NULL


def test_tile_struct_matches_the_header():
    import re
    header = open(os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                               "include", "nvfp4_w4a16.h")).read()
    body = re.search(r"typedef struct nvfp4_tile \{(.*?)\} nvfp4_tile_t;", header, re.S).group(1)
    names = re.findall(r"int (\w+);", body)
    assert names == [f for f, _ in nv.Tile._fields_]
    for name in ("KERNEL_AUTO", "KERNEL_PERSISTENT", "KERNEL_TILE", "KERNEL_SPLIT", "KERNEL_GENERIC",
                 "KERNEL_WHOLE"):
        value = int(re.search(r"NVFP4_%s = (\d+)" % name, header).group(1))
        assert getattr(nv, name) == value


def test_strerror_covers_every_status():
    seen = set()
    for st in range(-13, 1):
        msg = nv.strerror(st)
        assert msg and msg != "unknown status"
        seen.add(msg)
    assert len(seen) == 14
    assert nv.strerror(-99) == "unknown status"


def test_tile_info_depends_on_shape_only():
    for n, k in [(1024, 1024), (4096, 4096), (12288, 4096), (151552, 4096), (4096, 12288), (17, 256)]:
        info = nv.tile_info(n, k)
        assert f"N={n} K={k}" in info
        assert info == nv.tile_info(n, k)
        t = nv.table_tile(n, k)
        assert t.waves % t.split == 0 and t.mwaves in (0, 4, 6, 8)
    with pytest.raises(nv.Nvfp4Error):
        nv.tile_info(16, 100)
    buf = ctypes.create_string_buffer(8)
    assert nv._lib().nvfp4_tile_info(16, 256, buf, 8) == nv.ERR_BUFFER


def test_default_split_fills_the_chip():
    # Segment groups: enough 128-column workgroups for every one of 256 CUs,
    # at most one group per segment; a function of N (and K through waves).
    for n, k, split in [(4096, 2048, 8), (12288, 2048, 4), (32768, 4096, 1), (16384, 4096, 2),
                        (65536, 4096, 1), (151552, 4096, 1), (4096, 256, 2), (16, 1024, 8)]:
        t = nv.table_tile(n, k)
        assert t.split == min(split, t.waves), (n, k, t)


def test_builtin_table_entries():
    # Sweep-picked segment counts and groupings of the decode round's products
    # and of the row-invariance and fused-QKV configurations.
    for n, k, waves, split, mwaves in [(8192, 4096, 8, 4, 0), (4096, 8192, 8, 4, 4), (24576, 4096, 4, 1, 6),
                                       (4096, 12288, 8, 4, 4), (4096, 4096, 8, 4, 4), (12288, 4096, 8, 2, 8)]:
        t = nv.table_tile(n, k)
        assert (t.cols, t.waves, t.split, t.mwaves) == (16, waves, split, mwaves), (n, k, t)


def _tile_info_in_fresh_process(env_value, n=1024, k=1024):
    import subprocess, sys
    code = ("import verify_nvfp4_w4a16_amd as nv\n"
            "try:\n print(nv.tile_info(%d, %d))\n"
            "except nv.Nvfp4Error as e:\n print('status', e.status)\n" % (n, k))
    env = dict(os.environ)
    env.pop("NVFP4_TILES", None)
    if env_value is not None:
        env["NVFP4_TILES"] = env_value
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    out = subprocess.run([sys.executable, "-c", code], cwd=root, env=env,
                         capture_output=True, text=True, check=True)
    return out.stdout.strip()


def test_tile_override_file(tmp_path):
    # The table is read once per process, so each case runs in its own process.
    f = tmp_path / "tiles.txt"
    f.write_text("# N K cols waves unroll\n1024 1024 32 4 2\n")
    assert "cols=32 waves=4 unroll=2 split=1 mwaves=0" in _tile_info_in_fresh_process(str(f))
    f.write_text("1024 1024 32 4 2 2\n")
    assert "cols=32 waves=4 unroll=2 split=2 mwaves=0" in _tile_info_in_fresh_process(str(f))
    f.write_text("1024 1024 32 4 2 4 4  # comment\n")
    assert "cols=32 waves=4 unroll=2 split=4 mwaves=4" in _tile_info_in_fresh_process(str(f))
    for bad in ("1024 1024 32 4 2 8\n",          # more groups than segments
                "1024 1024 32 4 2 2 5\n",        # mwaves not 4, 6 or 8
                "1024 1024 32 4 2 2 8 1\n",      # too many fields
                "1024 1024 32 4\n",              # too few
                "1024 1024 32 4 2x\n",           # not an integer
                "1024 1024 4294967312 4 2\n"):   # out of range, not truncated
        f.write_text(bad)
        assert _tile_info_in_fresh_process(str(f)) == f"status {nv.ERR_TILEFILE}", bad
    f.write_text("1024 1024 48 4 2\n")
    assert _tile_info_in_fresh_process(str(f)) == f"status {nv.ERR_TILEFILE}"
    f.write_text("1024 1024 16 3 2\n")                # 3 does not divide 1024/128
    assert _tile_info_in_fresh_process(str(f)) == f"status {nv.ERR_TILEFILE}"
    assert _tile_info_in_fresh_process(str(tmp_path / "missing.txt")) == f"status {nv.ERR_TILEFILE}"
    assert "cols=32" not in _tile_info_in_fresh_process(None)


def test_build_rejects_kernels_that_spill():
    # The build reads the compiler's per-kernel resource report and refuses a
    # library in which any kernel spills registers to scratch memory.
    from verify_nvfp4_w4a16_amd import build
    report = "\n".join([
        "x.hip:1:1: remark: Function Name: _Z1av [-Rpass-analysis=kernel-resource-usage]",
        "x.hip:1:1: remark:     VGPRs: 80 [-Rpass-analysis=kernel-resource-usage]",
        "x.hip:1:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]",
        "x.hip:9:1: remark: Function Name: _Z1bv [-Rpass-analysis=kernel-resource-usage]",
        "x.hip:9:1: remark:     ScratchSize [bytes/lane]: 44 [-Rpass-analysis=kernel-resource-usage]",
    ])
    assert build.scratch_users(report) == [("_Z1bv", 44)]
    assert build.RESOURCE_REMARKS in " ".join([build.RESOURCE_REMARKS])


def test_read_probe_validates_before_any_hip_call():
    lib = ctypes.CDLL(nv.LIB_PATH)
    lib.nvfp4_read_probe.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64,
                                     ctypes.c_void_p, ctypes.c_void_p]
    a16, sink = 0x10000, 0x20000
    assert lib.nvfp4_read_probe(None, 16, None, 0, sink, None) == nv.ERR_NULL
    assert lib.nvfp4_read_probe(a16, 16, None, 0, None, None) == nv.ERR_NULL
    assert lib.nvfp4_read_probe(a16, 24, None, 0, sink, None) == nv.ERR_SHAPE
    assert lib.nvfp4_read_probe(a16, -16, None, 0, sink, None) == nv.ERR_SHAPE
    assert lib.nvfp4_read_probe(a16 + 8, 16, None, 0, sink, None) == nv.ERR_ALIGN
    assert lib.nvfp4_read_probe(a16, 16, None, 0, sink + 2, None) == nv.ERR_ALIGN
    assert lib.nvfp4_read_probe(None, 0, None, 0, sink, None) == nv.OK      # nothing to read


def test_group_record_layout_matches_the_header():
    # tests/host_check.cpp checks the C side (sizeof and offsetof) under the
    # sanitizers; this is the binding's side of the same layout.
    d = nv.GROUP_DTYPE
    assert d.itemsize == 40
    assert [d.fields[f][1] for f in ("x", "w_packed", "scales_e4m3", "y", "tensor_scale", "m")] == \
        [0, 8, 16, 24, 32, 36]


def test_fp8_pack_matches_oracle():
    g = workload.rng(8)
    for n, k in [(128, 128), (256, 384), (384, 1024)]:
        w = workload.weights_f32(n, k, n + k)
        w[:128, :128] *= np.float32(1e-30)                  # a block of tiny values
        w[128:256, 128:256] = 0.0 if n > 128 and k > 128 else w[128:256, 128:256]
        w[5, 7] = np.float32(3.0e4)                           # a dominant value in one block
        codes, scales = nv.fp8_pack(w)
        c2, s2 = oracle.quantize_fp8_ref(w)
        assert np.array_equal(scales, s2) and np.array_equal(codes, c2), (n, k)
    bad = np.zeros((128, 128), np.float32)
    bad[3, 3] = np.inf
    with pytest.raises(nv.Nvfp4Error):
        nv.fp8_pack(bad)
    with pytest.raises(nv.Nvfp4Error):
        nv.fp8_pack(np.zeros((100, 128), np.float32))
    assert nv.fp8_shape_ok(32, 128, 128) and not nv.fp8_shape_ok(33, 128, 128)
    assert not nv.fp8_shape_ok(1, 100, 128) and not nv.fp8_shape_ok(1, 128, 64)


def test_fp8_gemm_shape_contract():
    assert nv.fp8_gemm_shape_ok(0, 128, 128) and nv.fp8_gemm_shape_ok(33, 128, 128)
    assert nv.fp8_gemm_shape_ok(65535 * 128, 128, 128) and not nv.fp8_gemm_shape_ok(65535 * 128 + 1, 128, 128)
    assert not nv.fp8_gemm_shape_ok(-1, 128, 128) and not nv.fp8_gemm_shape_ok(64, 100, 128)
    assert not nv.fp8_gemm_shape_ok(64, 128, 64) and not nv.fp8_gemm_shape_ok(64, 128, (1 << 20) + 128)
    assert not nv.fp8_gemm_shape_ok(1 << 22, 1 << 19, 128)          # M * N above 2^40
