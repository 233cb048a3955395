"""C-ABI checks that need no GPU: the library loads, exports exactly the
entry points include/moe.h declares, and rejects bad arguments on the host
before any HIP call.  No compute call is made here."""

import ctypes
import os
import re
import subprocess

import pytest

from mixture_experts_moe_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B._LIB_PATH):
        from mixture_experts_moe_amd import build
        build.build()
    return B.lib()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"MOE_API\s+[\w\s\*]+?\b(moe_\w+)\s*\(", text)))


def test_header_declares_the_binding_entry_points():
    assert declared_functions() == sorted(B.ENTRY_POINTS)


def test_library_exports_exactly_the_declared_symbols(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", B._LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = sorted({l.split()[-1] for l in out.splitlines() if " T " in l})
    assert exported == declared_functions()


def desc(T=4, d=128, E=8, I=128, act=B.MOE_DTYPE_BF16, w=B.MOE_DTYPE_BF16, bm=0, q=None):
    return B.make_desc(T, d, E, I, act, w, bm, q)


E4 = B.MOE_DTYPE_E4M3FN


def ws_status(lib, dsc, k=2):
    n = ctypes.c_size_t()
    return lib.moe_workspace_bytes(ctypes.byref(dsc), k, 1, ctypes.byref(n))


@pytest.mark.parametrize("kw,k,status", [
    (dict(), 2, 0),
    (dict(T=-1), 2, -2),
    (dict(d=100), 2, -2),
    (dict(d=0), 2, -2),
    (dict(I=96), 2, -2),
    (dict(E=0), 1, -2),
    (dict(E=1025), 2, -2),
    (dict(), 0, -3),
    (dict(E=4), 5, -3),
    (dict(E=128), 65, -3),
    (dict(act=B.MOE_DTYPE_F32), 2, -4),
    (dict(act=B.MOE_DTYPE_E4M3FN, w=B.MOE_DTYPE_E4M3FN), 2, -4),
    (dict(act=B.MOE_DTYPE_F32, w=B.MOE_DTYPE_E4M3FN), 2, -4),
    (dict(bm=48), 2, -8),
    (dict(bm=256), 2, -8),                               # d = 128: the 256 GEMM needs d % 256 == 0
    (dict(d=256, bm=256), 2, 0),
    (dict(d=256, I=64, bm=256), 2, -8),                  # I % 128 != 0
    (dict(d=256, w=B.MOE_DTYPE_E4M3FN, bm=256), 2, -8),  # bf16 weights only
    (dict(bm=512), 2, -8),
    (dict(T=1 << 28), 8, -2),
    # the 256-token GEMM addresses an expert's W13 and x with 32-bit offsets
    (dict(T=1 << 18, d=4096, bm=256), 2, -8),          # 2*T*d = 2^31
    (dict(T=(1 << 18) - 64, d=4096, bm=256), 2, 0),
    (dict(d=1 << 15, I=1 << 15, bm=256), 2, -8),      # 4*I*d = 2^32
    # W8A8: bf16 x, e4m3fn weights, blocks of 256, d and I multiples of 256
    (dict(d=256, I=256, w=E4, q="mx_e4m3"), 2, 0),
    (dict(d=256, I=256, w=E4, bm=256, q="mx_e4m3"), 2, 0),
    (dict(d=256, I=256, q="mx_e4m3"), 2, -4),             # bf16 weights
    (dict(d=256, I=256, act=B.MOE_DTYPE_F32, w=B.MOE_DTYPE_F32, q="mx_e4m3"), 2, -4),
    (dict(d=256, I=256, w=E4, bm=128, q="mx_e4m3"), 2, -8),
    (dict(d=128, I=256, w=E4, q="mx_e4m3"), 2, -2),
    (dict(d=256, I=384, w=E4, q="mx_e4m3"), 2, -2),
    (dict(d=1 << 15, I=1 << 15, w=E4, q="mx_e4m3"), 2, -2),  # 2*I*d = 2^31
    (dict(T=1 << 19, d=4096, I=256, w=E4, q="mx_e4m3"), 2, -2),  # T*d = 2^31
    (dict(T=(1 << 19) - 64, d=4096, I=256, w=E4, q="mx_e4m3"), 2, 0),
])
def test_descriptor_validation(lib, kw, k, status):
    assert ws_status(lib, desc(**kw), k) == status


def test_schedule_field_validation(lib):
    d = desc()
    d.schedule = 3
    assert ws_status(lib, d) == -9
    d = desc()
    d.reserved = 1
    assert ws_status(lib, d) == -9
    with pytest.raises(ValueError):
        B.make_desc(4, 128, 8, 128, B.MOE_DTYPE_BF16, B.MOE_DTYPE_BF16, schedule="dynamic")
    for name in ("auto", "static", "queue"):
        assert ws_status(lib, B.make_desc(4, 128, 8, 128, B.MOE_DTYPE_BF16, B.MOE_DTYPE_BF16,
                                          schedule=name)) == 0


def test_queue_schedule_workspace(lib):
    """The queue's counters take workspace only where the 128-token GEMM runs
    with that schedule: not under the automatic schedule where blocks of 128
    take the register-token tile (bf16 weights, d = 256 is four of its K
    stages), but there where they do not (e4m3fn, two stages, below its
    three)."""
    def nbytes(bm, schedule, w=B.MOE_DTYPE_BF16):
        return B.moe_workspace_bytes(
            B.make_desc(512, 256, 8, 256, B.MOE_DTYPE_BF16, w, bm, None, schedule), 2, True)
    for w in (B.MOE_DTYPE_BF16, E4):
        assert nbytes(128, "queue", w) > nbytes(128, "static", w)
        assert nbytes(128, "queue", w) - nbytes(128, "static", w) <= 4096
    assert nbytes(128, "auto", B.MOE_DTYPE_BF16) == nbytes(128, "static", B.MOE_DTYPE_BF16)
    assert nbytes(128, "auto", E4) == nbytes(128, "queue", E4)
    assert nbytes(64, "queue") == nbytes(64, "static")
    assert nbytes(256, "queue") == nbytes(256, "static")


def test_unknown_act_quant_and_null_descriptor(lib):
    d = desc()
    d.act_quant = 2
    assert ws_status(lib, d) == -9
    with pytest.raises(ValueError):
        desc(q="mx_e5m2")
    n = ctypes.c_size_t()
    assert lib.moe_workspace_bytes(None, 2, 1, ctypes.byref(n)) == -1
    assert lib.moe_workspace_bytes(ctypes.byref(desc()), 2, 1, None) == -1


@pytest.mark.parametrize("T,E,k,bm", [(1, 8, 2, 16), (64, 8, 2, 64), (2048, 256, 8, 64),
                                     (5, 3, 3, 32), (4096, 8, 2, 128)])
def test_capacity_formula(lib, T, E, k, bm):
    got_bm, cap = B.moe_align_capacity(desc(T=T, E=E, bm=bm), k)
    A = T * k
    assert got_bm == bm
    assert cap == -(-(A + min(E, A) * (bm - 1)) // bm) * bm


def test_default_block_covers_a_decode_batch(lib):
    for T, want in [(1, 16), (8, 16), (16, 16), (17, 32), (32, 32), (64, 64), (65, 128)]:
        assert B.moe_align_capacity(desc(T=T), 2)[0] == want
    # LDS-streaming bf16 shapes: blocks of 16 while experts average at most
    # 8 slots (T = 32 at top-2 of 8), then blocks of 32 up to 64 tokens
    assert B.moe_align_capacity(desc(T=32, d=4096, I=14336), 2)[0] == 16
    assert B.moe_align_capacity(desc(T=33, d=4096, I=14336), 2)[0] == 32
    assert B.moe_align_capacity(desc(T=64, d=4096, I=14336), 2)[0] == 32
    assert B.moe_align_capacity(desc(T=64, d=4096, I=14336, w=B.MOE_DTYPE_E4M3FN), 2)[0] == 64
    # experts averaging >= 256 tokens with fitting bf16 shapes use the 256 GEMM
    assert B.moe_align_capacity(desc(T=4096, d=4096, I=14336), 2)[0] == 256
    assert B.moe_align_capacity(desc(T=4096, d=2880, I=2880), 2)[0] == 128
    assert B.moe_align_capacity(desc(T=4096, d=4096, I=14336, w=B.MOE_DTYPE_E4M3FN), 2)[0] == 128
    assert B.moe_align_capacity(desc(act=B.MOE_DTYPE_F32, w=B.MOE_DTYPE_F32), 2)[0] == 16
    # the W8A8 mode has one tile: blocks of 256 at any batch
    assert B.moe_align_capacity(desc(T=1, d=256, I=256, w=E4, q="mx_e4m3"), 2)[0] == 256


def test_workspace_grows_with_tokens(lib):
    sizes = [B.moe_workspace_bytes(desc(T=T), 2, True) for T in (1, 8, 64, 512)]
    assert sizes == sorted(sizes) and sizes[0] > 0
    assert B.moe_workspace_bytes(desc(T=0), 2, True) == 0
    assert B.moe_workspace_bytes(desc(T=64), 2, False) < B.moe_workspace_bytes(desc(T=64), 2, True)


FAKE = 1 << 20            # 16-byte aligned, never dereferenced: validation fails first


def fwd(lib, dsc, k=2, x=FAKE, wg=FAKE, w13=FAKE, w2=FAKE, out=FAKE, ws=FAKE, nbytes=1 << 40,
        scales=None):
    return lib.moe_forward(ctypes.byref(dsc), x, wg, w13, w2, k,
                           ctypes.byref(scales) if scales is not None else None, out, ws, nbytes,
                           None)


def test_forward_rejects_before_any_hip_call(lib):
    d = desc()
    assert fwd(lib, d, x=None) == -1
    assert fwd(lib, d, wg=None) == -1
    assert fwd(lib, d, out=None) == -1
    assert fwd(lib, d, x=FAKE + 8) == -5
    assert fwd(lib, d, w13=FAKE + 4) == -5
    assert fwd(lib, d, ws=None) == -6
    assert fwd(lib, d, nbytes=16) == -6
    assert fwd(lib, d, ws=FAKE + 16) == -5        # workspace must be 256-byte aligned
    assert fwd(lib, d, k=9) == -3
    # T = 0 returns OK without looking at any pointer
    assert fwd(lib, desc(T=0), x=None, wg=None, w13=None, w2=None, out=None, ws=None, nbytes=0) == 0


def test_scale_validation(lib):
    d8 = desc(w=B.MOE_DTYPE_E4M3FN)
    assert fwd(lib, d8) == -1                                      # fp8 needs scales
    sc = B.moe_scales(B.MOE_SCALE_NONE, 0, FAKE, FAKE)
    assert fwd(lib, d8, scales=sc) == -4
    sc = B.moe_scales(B.MOE_SCALE_PER_CHANNEL, 0, None, FAKE)
    assert fwd(lib, d8, scales=sc) == -1
    sc = B.moe_scales(B.MOE_SCALE_PER_TENSOR, 0, FAKE + 4, FAKE)
    assert fwd(lib, d8, scales=sc) == -5
    sc = B.moe_scales(B.MOE_SCALE_PER_CHANNEL, 1, FAKE, FAKE)
    assert fwd(lib, d8, scales=sc) == -9
    sc = B.moe_scales(B.MOE_SCALE_PER_CHANNEL, 0, FAKE, FAKE)
    assert fwd(lib, desc(), scales=sc) == -4                       # bf16 weights take no scales


def test_stage_entry_points_validate(lib):
    d = desc()
    P = ctypes.c_void_p
    assert lib.moe_route(ctypes.byref(d), None, FAKE, 2, FAKE, FAKE, FAKE, None) == -1
    assert lib.moe_route(ctypes.byref(d), FAKE, FAKE, 0, FAKE, FAKE, FAKE, None) == -3
    assert lib.moe_route_logits(ctypes.byref(d), FAKE, 2, FAKE, None, None) == -1
    assert lib.moe_align(ctypes.byref(d), FAKE, 2, FAKE, FAKE, FAKE + 2, FAKE, None) == -5
    assert lib.moe_expert_ffn(ctypes.byref(d), FAKE, FAKE, FAKE, 2, None, FAKE, FAKE, FAKE, FAKE,
                              FAKE, FAKE, 0, None) == -6
    assert lib.moe_route(ctypes.byref(desc(T=0)), None, None, 2, None, None, None, None) == 0


def test_quantize_act_validates(lib):
    q = lib.moe_quantize_act
    d8 = desc(d=256, I=256, w=E4, q="mx_e4m3")
    assert q(ctypes.byref(d8), None, FAKE, FAKE, None) == -1
    assert q(ctypes.byref(d8), FAKE, FAKE, FAKE + 8, None) == -5
    assert q(ctypes.byref(desc(d=256, I=256, w=E4)), FAKE, FAKE, FAKE, None) == -9  # not W8A8
    assert q(ctypes.byref(desc(d=128, I=256, w=E4, q="mx_e4m3")), FAKE, FAKE, FAKE, None) == -2
    assert q(None, FAKE, FAKE, FAKE, None) == -1
    assert q(ctypes.byref(desc(T=0, d=256, I=256, w=E4, q="mx_e4m3")), None, None, None, None) == 0


def test_route_align_and_graph_validate(lib):
    d = desc()
    ra = lib.moe_route_align
    assert ra(ctypes.byref(d), None, FAKE, 2, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == -1
    assert ra(ctypes.byref(d), FAKE, FAKE, 9, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == -3
    assert ra(ctypes.byref(d), FAKE, FAKE, 2, FAKE, FAKE, FAKE, FAKE + 4, FAKE, FAKE, FAKE,
              None) == -5
    assert ra(ctypes.byref(desc(T=0)), None, None, 2, None, None, None, None, None, None, None,
              None) == 0
    h = ctypes.c_void_p(12345)
    gc = lib.moe_graph_create
    assert gc(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, 2, None, FAKE, FAKE, 1 << 40, None) == -1
    assert gc(ctypes.byref(d), None, FAKE, FAKE, FAKE, 2, None, FAKE, FAKE, 1 << 40,
              ctypes.byref(h)) == -1
    assert h.value is None                       # NULL on error
    assert gc(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, 2, None, FAKE, FAKE, 16,
              ctypes.byref(h)) == -6
    assert gc(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, 2, None, FAKE, FAKE + 16, 1 << 40,
              ctypes.byref(h)) == -5
    # T = 0: a handle whose replay does nothing (no HIP call anywhere)
    assert gc(ctypes.byref(desc(T=0)), None, None, None, None, 2, None, None, None, 0,
              ctypes.byref(h)) == 0
    assert h.value
    assert lib.moe_graph_launch(h, None) == 0
    assert lib.moe_graph_destroy(h) == 0
    assert lib.moe_graph_launch(None, None) == -1
    assert lib.moe_graph_destroy(None) == 0


BENCH_HEADER = os.path.join(ROOT, "include", "moe_bench.h")


def test_bench_library_exports_and_validates():
    from mixture_experts_moe_amd import build
    if not os.path.exists(B._BENCH_LIB_PATH):
        build.build_bench()
    declared = sorted(set(re.findall(r"MOE_BENCH_API\s+[\w\s\*]+?\b(moe_bench_\w+)\s*\(",
                                     open(BENCH_HEADER).read())))
    assert declared == sorted(B.BENCH_ENTRY_POINTS)
    out = subprocess.run(["nm", "-D", "--defined-only", B._BENCH_LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    assert sorted({l.split()[-1] for l in out.splitlines() if " T " in l}) == declared
    L = B.bench_lib()
    r = ctypes.c_double()
    assert L.moe_bench_hbm_read(None, 1 << 20, 3, ctypes.byref(r), None) == -1
    assert L.moe_bench_hbm_read(FAKE, 1 << 20, 3, None, None) == -1
    assert L.moe_bench_hbm_read(FAKE, (1 << 20) + 1024, 3, ctypes.byref(r), None) == -9
    assert L.moe_bench_hbm_read(FAKE, 1 << 20, 1, ctypes.byref(r), None) == -9
    assert L.moe_bench_hbm_read(FAKE + 8, 1 << 20, 3, ctypes.byref(r), None) == -9
    assert L.moe_bench_mfma_bf16(100, 3, None, None) == -1
    assert L.moe_bench_mfma_bf16(1, 3, ctypes.byref(r), None) == -9
    assert L.moe_bench_mfma_bf16(100, 1, ctypes.byref(r), None) == -9
    assert L.moe_bench_mfma_fp8(100, 3, None, None) == -1
    assert L.moe_bench_mfma_fp8(1, 3, ctypes.byref(r), None) == -9
    assert L.moe_bench_mfma_fp8(100, 1, ctypes.byref(r), None) == -9
    assert L.moe_bench_fp8_dot(None, FAKE, FAKE, FAKE, 4, None) == -1
    assert L.moe_bench_fp8_dot(FAKE, FAKE, FAKE, None, 4, None) == -1
    assert L.moe_bench_fp8_dot(FAKE, FAKE, FAKE, FAKE, 0, None) == -9
    assert L.moe_bench_fp8_dot(FAKE + 8, FAKE, FAKE, FAKE, 4, None) == -9


def test_strerror_and_names(lib):
    for code in range(0, -11, -1):
        s = B.strerror(code)
        assert s and s != "unknown status"
    assert B.strerror(-99) == "unknown status"
    names = [B.moe_kernel_name(i) for i in range(B.MOE_KERNEL_COUNT)]
    assert names == ["route_logits", "route_topk", "align", "ffn13", "ffn2", "combine",
                     "quant_x", "ffn_fused"]
    assert B.moe_kernel_name(99) == ""


def test_timing_collect_without_work(lib):
    B.moe_timing_enable(True)
    t = B.moe_timing_collect(reset=True)
    assert all(v == (0.0, 0) for v in t.values())
    B.moe_timing_enable(False)


def test_noalloc_forward_rejects_before_any_hip_call(lib):
    """moe_forward_noalloc checks its arguments and the size of its static
    workspace on the host before its first HIP call (the device lookup of
    that array), so these return without a GPU."""
    def call(dsc, k=2, x=FAKE, wg=FAKE, w13=FAKE, w2=FAKE, out=FAKE, scales=None):
        return lib.moe_forward_noalloc(ctypes.byref(dsc), x, wg, w13, w2, k,
                                       ctypes.byref(scales) if scales is not None else None,
                                       out, None)
    d = desc()
    assert call(d, x=None) == -1
    assert call(d, out=None) == -1
    assert call(d, w2=FAKE + 8) == -5
    assert call(d, k=9) == -3
    assert call(desc(w=B.MOE_DTYPE_E4M3FN)) == -1                  # fp8 needs scales
    assert call(desc(T=0), x=None, wg=None, w13=None, w2=None, out=None) == 0
    # a layer whose workspace exceeds the array: the size error, before any HIP call
    big = desc(T=20000, d=512, I=512)
    n = ctypes.c_size_t()
    assert lib.moe_workspace_bytes(ctypes.byref(big), 2, 1, ctypes.byref(n)) == 0
    assert n.value > B.MOE_NOALLOC_WORKSPACE_BYTES
    assert call(big) == B.MOE_ERR_NOALLOC_SIZE == -10
    assert "static" in B.strerror(-10)
