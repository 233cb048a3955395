"""ctypes binding of the fused MoE C ABI (include/moe.h).

Argument marshalling only: every function takes torch tensors, checks their
shapes, dtypes and devices, and calls the C entry point of the same name with
raw device pointers and a HIP stream (the one given, else torch's current
stream of the tensors' device).  Tensors the binding allocates (outputs,
workspace) are allocated on that stream, so torch's caching allocator only
reuses their memory for work ordered after these kernels.  All computation happens in
the HIP kernels of ``libmoe.so``; there is no fallback of any kind, and if
the library is missing the first call raises.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple

import torch

# MOE_LIBRARY may name another build of the same library (e.g. a tuning variant).
_LIB_PATH = os.environ.get("MOE_LIBRARY") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "libmoe.so")

MOE_DTYPE_F32 = 0
MOE_DTYPE_BF16 = 1
MOE_DTYPE_E4M3FN = 2
MOE_SCALE_NONE = 0
MOE_SCALE_PER_TENSOR = 1
MOE_SCALE_PER_CHANNEL = 2
MOE_ACT_AS_IS = 0
MOE_ACT_MX_E4M3 = 1
MOE_SCHED_AUTO = 0
MOE_SCHED_STATIC = 1
MOE_SCHED_QUEUE = 2
MOE_KERNEL_COUNT = 8

ENTRY_POINTS = (
    "moe_align_capacity", "moe_workspace_bytes", "moe_forward", "moe_route",
    "moe_route_logits", "moe_align", "moe_route_align", "moe_expert_ffn",
    "moe_quantize_act", "moe_graph_create", "moe_graph_launch", "moe_graph_destroy", "moe_strerror",
    "moe_timing_enable", "moe_timing_collect", "moe_kernel_name", "moe_forward_noalloc",
)
MOE_ERR_NOALLOC_SIZE = -10
MOE_NOALLOC_WORKSPACE_BYTES = 64 << 20


class moe_desc(ctypes.Structure):
    _fields_ = [("num_tokens", ctypes.c_int64), ("hidden", ctypes.c_int64),
                ("num_experts", ctypes.c_int64), ("intermediate", ctypes.c_int64),
                ("act_dtype", ctypes.c_int32), ("weight_dtype", ctypes.c_int32),
                ("block_m", ctypes.c_int32), ("act_quant", ctypes.c_int32),
                ("schedule", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class moe_scales(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("w13", ctypes.c_void_p), ("w2", ctypes.c_void_p)]


class MoEError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: {strerror(status)} (status {status})")


_lib = None


def lib() -> ctypes.CDLL:
    """Load libmoe.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is not built; run `python -m mixture_experts_moe_amd.build`")
    L = ctypes.CDLL(_LIB_PATH)
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
    D = ctypes.POINTER(moe_desc)
    S = ctypes.POINTER(moe_scales)
    sig = {
        "moe_align_capacity": (I32, [D, I32, ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(I64)]),
        "moe_workspace_bytes": (I32, [D, I32, I32, ctypes.POINTER(SZ)]),
        "moe_forward": (I32, [D, P, P, P, P, I32, S, P, P, SZ, P]),
        "moe_forward_noalloc": (I32, [D, P, P, P, P, I32, S, P, P]),
        "moe_route": (I32, [D, P, P, I32, P, P, P, P]),
        "moe_route_logits": (I32, [D, P, I32, P, P, P]),
        "moe_align": (I32, [D, P, I32, P, P, P, P, P]),
        "moe_route_align": (I32, [D, P, P, I32, P, P, P, P, P, P, P, P]),
        "moe_graph_create": (I32, [D, P, P, P, P, I32, S, P, P, SZ, ctypes.POINTER(P)]),
        "moe_graph_launch": (I32, [P, P]),
        "moe_graph_destroy": (I32, [P]),
        "moe_expert_ffn": (I32, [D, P, P, P, I32, S, P, P, P, P, P, P, SZ, P]),
        "moe_quantize_act": (I32, [D, P, P, P, P]),
        "moe_strerror": (ctypes.c_char_p, [I32]),
        "moe_timing_enable": (I32, [I32]),
        "moe_timing_collect": (I32, [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(I64), I32]),
        "moe_kernel_name": (ctypes.c_char_p, [I32]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _lib = L
    return L


# ------------------------------------------------------------ attainable-rate probes

BENCH_ENTRY_POINTS = ("moe_bench_hbm_read", "moe_bench_mfma_bf16", "moe_bench_mfma_fp8",
                      "moe_bench_fp8_dot")
_BENCH_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe_bench.so")
_bench_lib = None


def bench_lib() -> ctypes.CDLL:
    """Load libmoe_bench.so (once).  Raises if it has not been built."""
    global _bench_lib
    if _bench_lib is not None:
        return _bench_lib
    if not os.path.exists(_BENCH_LIB_PATH):
        raise RuntimeError(f"{_BENCH_LIB_PATH} is not built; run `python -m mixture_experts_moe_amd.build`")
    L = ctypes.CDLL(_BENCH_LIB_PATH)
    P, I32, SZ, D = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.POINTER(ctypes.c_double)
    L.moe_bench_hbm_read.restype = I32
    L.moe_bench_hbm_read.argtypes = [P, SZ, I32, D, P]
    L.moe_bench_mfma_bf16.restype = I32
    L.moe_bench_mfma_bf16.argtypes = [I32, I32, D, P]
    L.moe_bench_mfma_fp8.restype = I32
    L.moe_bench_mfma_fp8.argtypes = [I32, I32, D, P]
    L.moe_bench_fp8_dot.restype = I32
    L.moe_bench_fp8_dot.argtypes = [P, P, P, P, I32, P]
    _bench_lib = L
    return L


def bench_hbm_read(buf: torch.Tensor, reps: int = 5, stream=None) -> float:
    """Attainable streaming-read rate (GB/s) over the device buffer `buf`."""
    dev = _dev(buf)
    r = ctypes.c_double()
    _check("moe_bench_hbm_read", bench_lib().moe_bench_hbm_read(
        _ptr(buf), buf.numel() * buf.element_size(), int(reps), ctypes.byref(r),
        _stream(dev, stream)))
    return r.value


def bench_mfma_bf16(iters: int = 4096, reps: int = 4, device="cuda", stream=None) -> float:
    """Attainable bf16 MFMA rate (TFLOP/s) of an LDS-fed loop on random data."""
    dev = torch.device(device)
    r = ctypes.c_double()
    _check("moe_bench_mfma_bf16", bench_lib().moe_bench_mfma_bf16(
        int(iters), int(reps), ctypes.byref(r), _stream(dev, stream)))
    return r.value


def bench_mfma_fp8(iters: int = 4096, reps: int = 4, device="cuda", stream=None) -> float:
    """Attainable e4m3fn (block-scaled) MFMA rate (TFLOP/s) of the W8A8 tile's
    LDS-fed loop on random codes."""
    dev = torch.device(device)
    r = ctypes.c_double()
    _check("moe_bench_mfma_fp8", bench_lib().moe_bench_mfma_fp8(
        int(iters), int(reps), ctypes.byref(r), _stream(dev, stream)))
    return r.value


def bench_fp8_dot(a: torch.Tensor, b: torch.Tensor, c: torch.Tensor, stream=None) -> torch.Tensor:
    """c[t] + A[t] . B[t] for e4m3fn code rows a, b [n, 128] (uint8) and
    fp32 c [n], as the scaled fp8 MFMA computes it (unit block scales)."""
    dev = _dev(a, b, c)
    if a.dtype != torch.uint8 or b.dtype != torch.uint8 or c.dtype != torch.float32:
        raise TypeError("a, b must be uint8 codes and c float32")
    n = a.shape[0]
    if tuple(a.shape) != (n, 128) or tuple(b.shape) != (n, 128) or tuple(c.shape) != (n,):
        raise ValueError("a, b must be [n, 128] and c [n]")
    out = torch.empty((n, 256), dtype=torch.float32, device=dev)
    _check("moe_bench_fp8_dot", bench_lib().moe_bench_fp8_dot(
        _ptr(a), _ptr(b), _ptr(c), _ptr(out), int(n), _stream(dev, stream)))
    if not bool((out == out[:, :1]).all()):
        raise RuntimeError("moe_bench_fp8_dot: the tile's 256 outputs differ")
    return out[:, 0].contiguous()


def strerror(status: int) -> str:
    return lib().moe_strerror(int(status)).decode()


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise MoEError(fn, status)


# ------------------------------------------------------------ marshalling

def _act_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return MOE_DTYPE_F32
    if t.dtype == torch.bfloat16:
        return MOE_DTYPE_BF16
    raise TypeError(f"activations must be float32 or bfloat16, got {t.dtype}")


def _w_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return MOE_DTYPE_F32
    if t.dtype == torch.bfloat16:
        return MOE_DTYPE_BF16
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return MOE_DTYPE_E4M3FN
    raise TypeError(f"weights must be float32, bfloat16 or e4m3fn bytes, got {t.dtype}")


def _act_quant_code(act_quant: Optional[str]) -> int:
    if act_quant is None:
        return MOE_ACT_AS_IS
    if act_quant == "mx_e4m3":
        return MOE_ACT_MX_E4M3
    raise ValueError(f"act_quant must be None or 'mx_e4m3', got {act_quant!r}")


_SCHEDULES = {"auto": MOE_SCHED_AUTO, "static": MOE_SCHED_STATIC, "queue": MOE_SCHED_QUEUE}


def _schedule_code(schedule: str) -> int:
    if schedule not in _SCHEDULES:
        raise ValueError(f"schedule must be one of {sorted(_SCHEDULES)}, got {schedule!r}")
    return _SCHEDULES[schedule]


def make_desc(T: int, d: int, E: int, I: int, act_dtype: int, weight_dtype: int,
              block_m: int = 0, act_quant: Optional[str] = None,
              schedule: str = "auto") -> moe_desc:
    return moe_desc(int(T), int(d), int(E), int(I), int(act_dtype), int(weight_dtype),
                    int(block_m), _act_quant_code(act_quant), _schedule_code(schedule), 0)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev(*ts: Optional[torch.Tensor]) -> torch.device:
    dev = None
    for t in ts:
        if t is None:
            continue
        if t.device.type != "cuda":
            raise ValueError("all tensors must be on the GPU")
        if not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError("all tensors must be on one device")
    return dev


def _stream(dev: torch.device, stream=None):
    s = stream if stream is not None else torch.cuda.current_stream(dev)
    return ctypes.c_void_p(s.cuda_stream)


def _scales(w13: torch.Tensor, scales) -> Optional[moe_scales]:
    if _w_code(w13) != MOE_DTYPE_E4M3FN:
        if scales is not None:
            raise ValueError("scales are only for e4m3fn weights")
        return None
    if scales is None:
        raise ValueError("e4m3fn weights need (s13, s2) scales")
    s13, s2 = scales
    if s13.dtype != torch.float32 or s2.dtype != torch.float32:
        raise TypeError("scales must be float32")
    if _dev(w13, s13, s2) != w13.device:
        raise ValueError("scales must be on the weights' device")
    E, two_i, d = w13.shape
    if s13.dim() == 2:
        mode = MOE_SCALE_PER_CHANNEL
        if tuple(s13.shape) != (E, two_i) or tuple(s2.shape) != (E, d):
            raise ValueError(f"per-channel scales must be [{E}, {two_i}] and [{E}, {d}]")
    else:
        mode = MOE_SCALE_PER_TENSOR
        if tuple(s13.shape) != (E,) or tuple(s2.shape) != (E,):
            raise ValueError(f"per-tensor scales must be [{E}] and [{E}]")
    return moe_scales(mode, 0, s13.data_ptr(), s2.data_ptr())


def _shapes(x, w_gate, w13, w2):
    """(T, d, E, I) from the tensors' shapes; raises before any launch when
    shapes or dtypes do not fit together (metadata only: no device access)."""
    if x.dim() != 2:
        raise ValueError(f"x must be [T, d], got shape {tuple(x.shape)}")
    T, d = x.shape
    if w13.dim() != 3 or w2.dim() != 3:
        raise ValueError("w13 must be [E, 2I, d] and w2 [E, d, I]")
    if _w_code(w2) != _w_code(w13) or w2.element_size() != w13.element_size():
        raise TypeError(f"w13 and w2 must have one weight format, got {w13.dtype} and {w2.dtype}")
    E, twoI, d13 = w13.shape
    I = twoI // 2
    if d13 != d or twoI != 2 * I or tuple(w2.shape) != (E, d, I):
        raise ValueError(f"shape mismatch: x {tuple(x.shape)}, w13 {tuple(w13.shape)}, w2 {tuple(w2.shape)}")
    if w_gate is not None:
        if w_gate.dtype != torch.float32 or tuple(w_gate.shape) != (E, d):
            raise ValueError(f"w_gate must be float32 [{E}, {d}]")
    return T, d, E, I


def _launch_stream(dev: torch.device, stream=None):
    """The torch stream the kernels are enqueued on."""
    return stream if stream is not None else torch.cuda.current_stream(dev)


def _alloc(shape, dtype, dev, stream) -> torch.Tensor:
    """A new device tensor owned by `stream` in torch's caching allocator, so
    that once it is dropped its memory is only handed to later work on that
    same stream, i.e. after the kernels enqueued here have used it."""
    with torch.cuda.stream(stream):
        return torch.empty(shape, dtype=dtype, device=dev)


def _workspace(nbytes: int, dev, workspace: Optional[torch.Tensor], stream) -> torch.Tensor:
    if workspace is not None:
        if workspace.numel() * workspace.element_size() < nbytes:
            raise ValueError("workspace too small")
        return workspace
    return _alloc((max(nbytes, 1),), torch.uint8, dev, stream)


def _check_out(out: torch.Tensor, x: torch.Tensor) -> None:
    if tuple(out.shape) != tuple(x.shape) or out.dtype != x.dtype:
        raise ValueError(f"out must match x in shape and dtype: out {tuple(out.shape)} "
                         f"{out.dtype}, x {tuple(x.shape)} {x.dtype}")


def _check_routing(T: int, top_k: int, topk_w: torch.Tensor, sorted_ids: torch.Tensor,
                   block_expert: torch.Tensor, num_padded: torch.Tensor, cap: int,
                   bm: int) -> None:
    """The routing tensors moe_expert_ffn reads: gates fp32 [T, k], the
    regrouped layout int32 and at least as long as the capacity."""
    if topk_w.dtype != torch.float32 or tuple(topk_w.shape) != (T, top_k):
        raise ValueError(f"topk_w must be float32 [{T}, {top_k}], got {topk_w.dtype} "
                         f"{tuple(topk_w.shape)}")
    for name, t in (("sorted_ids", sorted_ids), ("block_expert", block_expert),
                    ("num_padded", num_padded)):
        if t.dtype != torch.int32:
            raise TypeError(f"{name} must be int32, got {t.dtype}")
    if sorted_ids.numel() < cap or block_expert.numel() < cap // bm:
        raise ValueError("sorted_ids / block_expert smaller than the layout capacity")
    if num_padded.numel() < 1:
        raise ValueError("num_padded must hold one int32")


# ------------------------------------------------------------ entry points

def moe_align_capacity(desc: moe_desc, top_k: int) -> Tuple[int, int]:
    """(block_m, capacity) of the regrouped layout for `desc`."""
    bm = ctypes.c_int32()
    cap = ctypes.c_int64()
    _check("moe_align_capacity", lib().moe_align_capacity(ctypes.byref(desc), int(top_k),
                                                         ctypes.byref(bm), ctypes.byref(cap)))
    return bm.value, cap.value


def moe_workspace_bytes(desc: moe_desc, top_k: int, with_routing: bool = True) -> int:
    n = ctypes.c_size_t()
    _check("moe_workspace_bytes", lib().moe_workspace_bytes(ctypes.byref(desc), int(top_k),
                                                           int(bool(with_routing)), ctypes.byref(n)))
    return n.value


def moe_forward(x: torch.Tensor, w_gate: torch.Tensor, w13: torch.Tensor, w2: torch.Tensor,
                top_k: int, scales: Optional[Sequence[torch.Tensor]] = None,
                out: Optional[torch.Tensor] = None, *, block_m: int = 0,
                workspace: Optional[torch.Tensor] = None, stream=None,
                act_quant: Optional[str] = None, schedule: str = "auto") -> torch.Tensor:
    """out [T, d] = fused MoE layer of x (same dtype as x).  act_quant="mx_e4m3"
    selects the W8A8 mode (e4m3fn weights; x and h block-scaled e4m3fn);
    schedule ("auto", "static", "queue") how the 128-token-block expert
    kernels hand out their tiles."""
    T, d, E, I = _shapes(x, w_gate, w13, w2)
    if out is not None:
        _check_out(out, x)
    dev = _dev(x, w_gate, w13, w2, out)
    desc = make_desc(T, d, E, I, _act_code(x), _w_code(w13), block_m, act_quant, schedule)
    sc = _scales(w13, scales)
    s = _launch_stream(dev, stream)
    if out is None:
        out = _alloc((T, d), x.dtype, dev, s)
    nbytes = moe_workspace_bytes(desc, top_k, True)
    ws = _workspace(nbytes, dev, workspace, s)
    st = lib().moe_forward(ctypes.byref(desc), _ptr(x), _ptr(w_gate), _ptr(w13), _ptr(w2),
                           int(top_k), ctypes.byref(sc) if sc is not None else None, _ptr(out),
                           _ptr(ws), nbytes, ctypes.c_void_p(s.cuda_stream))
    _check("moe_forward", st)
    return out


def moe_forward_noalloc(x: torch.Tensor, w_gate: torch.Tensor, w13: torch.Tensor,
                        w2: torch.Tensor, top_k: int, out: torch.Tensor,
                        scales: Optional[Sequence[torch.Tensor]] = None, *, block_m: int = 0,
                        stream=None, act_quant: Optional[str] = None,
                        schedule: str = "auto") -> torch.Tensor:
    """moe_forward into the caller's `out` with the library's static
    workspace (the C entry point allocates nothing; nor does this wrapper).
    Raises MoEError (status MOE_ERR_NOALLOC_SIZE) when the layer needs more
    than MOE_NOALLOC_WORKSPACE_BYTES of workspace.  Calls that may overlap on
    one GPU share that workspace and race."""
    T, d, E, I = _shapes(x, w_gate, w13, w2)
    _check_out(out, x)
    dev = _dev(x, w_gate, w13, w2, out)
    desc = make_desc(T, d, E, I, _act_code(x), _w_code(w13), block_m, act_quant, schedule)
    sc = _scales(w13, scales)
    s = _launch_stream(dev, stream)
    st = lib().moe_forward_noalloc(ctypes.byref(desc), _ptr(x), _ptr(w_gate), _ptr(w13),
                                   _ptr(w2), int(top_k),
                                   ctypes.byref(sc) if sc is not None else None, _ptr(out),
                                   ctypes.c_void_p(s.cuda_stream))
    _check("moe_forward_noalloc", st)
    return out


def moe_route(x: torch.Tensor, w_gate: torch.Tensor, top_k: int, *, stream=None):
    """(logits [T,E] fp32, topk_ids [T,k] int32, topk_w [T,k] fp32)."""
    dev = _dev(x, w_gate)
    s = _launch_stream(dev, stream)
    T, d = x.shape
    E = w_gate.shape[0]
    if w_gate.dtype != torch.float32 or w_gate.shape[1] != d:
        raise ValueError("w_gate must be float32 [E, d]")
    desc = make_desc(T, d, E, 64, _act_code(x), _act_code(x))
    logits = _alloc((T, E), torch.float32, dev, s)
    ids = _alloc((T, top_k), torch.int32, dev, s)
    w = _alloc((T, top_k), torch.float32, dev, s)
    _check("moe_route", lib().moe_route(ctypes.byref(desc), _ptr(x), _ptr(w_gate), int(top_k),
                                        _ptr(logits), _ptr(ids), _ptr(w), ctypes.c_void_p(s.cuda_stream)))
    return logits, ids, w


def moe_route_logits(logits: torch.Tensor, top_k: int, *, stream=None):
    """(topk_ids [T,k] int32, topk_w [T,k] fp32) from given fp32 logits [T,E]."""
    dev = _dev(logits)
    s = _launch_stream(dev, stream)
    if logits.dtype != torch.float32 or logits.dim() != 2:
        raise ValueError("logits must be float32 [T, E]")
    T, E = logits.shape
    desc = make_desc(T, 64, E, 64, MOE_DTYPE_F32, MOE_DTYPE_F32)
    ids = _alloc((T, top_k), torch.int32, dev, s)
    w = _alloc((T, top_k), torch.float32, dev, s)
    _check("moe_route_logits", lib().moe_route_logits(ctypes.byref(desc), _ptr(logits), int(top_k),
                                                      _ptr(ids), _ptr(w), ctypes.c_void_p(s.cuda_stream)))
    return ids, w


def moe_quantize_act(x: torch.Tensor, *, stream=None):
    """W8A8 activation quantisation of bf16 x [T, d]: (codes [T, d] uint8
    e4m3fn bytes, exps [T, d/32] uint8 E8M0 bytes, scale 2^(byte - 127))."""
    dev = _dev(x)
    s = _launch_stream(dev, stream)
    if x.dtype != torch.bfloat16 or x.dim() != 2:
        raise ValueError("x must be bfloat16 [T, d]")
    T, d = x.shape
    inter = 256
    desc = make_desc(T, d, 1, inter, MOE_DTYPE_BF16, MOE_DTYPE_E4M3FN, 0, "mx_e4m3")
    codes = _alloc((T, d), torch.uint8, dev, s)
    exps = _alloc((T, d // 32), torch.uint8, dev, s)
    _check("moe_quantize_act", lib().moe_quantize_act(ctypes.byref(desc), _ptr(x), _ptr(codes),
                                                      _ptr(exps), ctypes.c_void_p(s.cuda_stream)))
    return codes, exps


def moe_align(topk_ids: torch.Tensor, num_experts: int, *, block_m: int = 0, hidden: int = 64,
              intermediate: int = 64, act_dtype: int = MOE_DTYPE_BF16,
              weight_dtype: int = MOE_DTYPE_BF16, stream=None, act_quant: Optional[str] = None):
    """Regroup slots by expert: (counts [E], sorted_ids [cap], block_expert [cap/B],
    num_padded [1], block_m).  The default block_m depends on the whole
    descriptor, so pass the layer's dims/dtypes/act_quant to get the one
    moe_forward uses."""
    dev = _dev(topk_ids)
    s = _launch_stream(dev, stream)
    if topk_ids.dtype != torch.int32 or topk_ids.dim() != 2:
        raise ValueError("topk_ids must be int32 [T, k]")
    T, k = topk_ids.shape
    desc = make_desc(T, hidden, num_experts, intermediate, act_dtype, weight_dtype, block_m,
                     act_quant)
    B, cap = moe_align_capacity(desc, k)
    counts = _alloc(num_experts, torch.int32, dev, s)
    sorted_ids = _alloc(max(cap, 1), torch.int32, dev, s)
    block_expert = _alloc(max(cap // B, 1), torch.int32, dev, s)
    num_padded = _alloc((4,), torch.int32, dev, s)
    _check("moe_align", lib().moe_align(ctypes.byref(desc), _ptr(topk_ids), int(k), _ptr(counts),
                                        _ptr(sorted_ids), _ptr(block_expert), _ptr(num_padded),
                                        ctypes.c_void_p(s.cuda_stream)))
    return counts, sorted_ids[:cap], block_expert[:cap // B], num_padded[:1], B


def moe_route_align(x: torch.Tensor, w_gate: torch.Tensor, top_k: int, *, intermediate: int = 64,
                    weight_dtype: int = MOE_DTYPE_BF16, block_m: int = 0, stream=None):
    """Routing then regrouping in one call: (logits, topk_ids, topk_w, counts,
    sorted_ids, block_expert, num_padded, block_m), as moe_route followed by
    moe_align with the same descriptor (pass the layer's intermediate size
    and weight dtype to get the block size moe_forward uses)."""
    dev = _dev(x, w_gate)
    s = _launch_stream(dev, stream)
    T, d = x.shape
    E = w_gate.shape[0]
    if w_gate.dtype != torch.float32 or w_gate.shape[1] != d:
        raise ValueError("w_gate must be float32 [E, d]")
    desc = make_desc(T, d, E, intermediate, _act_code(x), weight_dtype, block_m)
    B, cap = moe_align_capacity(desc, top_k)
    logits = _alloc((T, E), torch.float32, dev, s)
    ids = _alloc((T, top_k), torch.int32, dev, s)
    w = _alloc((T, top_k), torch.float32, dev, s)
    counts = _alloc(E, torch.int32, dev, s)
    sorted_ids = _alloc(max(cap, 1), torch.int32, dev, s)
    block_expert = _alloc(max(cap // B, 1), torch.int32, dev, s)
    num_padded = _alloc((4,), torch.int32, dev, s)
    _check("moe_route_align", lib().moe_route_align(
        ctypes.byref(desc), _ptr(x), _ptr(w_gate), int(top_k), _ptr(logits), _ptr(ids), _ptr(w),
        _ptr(counts), _ptr(sorted_ids), _ptr(block_expert), _ptr(num_padded),
        ctypes.c_void_p(s.cuda_stream)))
    return logits, ids, w, counts, sorted_ids[:cap], block_expert[:cap // B], num_padded[:1], B


class MoeGraph:
    """moe_forward recorded once into a HIP graph (moe_graph_create) and
    replayed with one launch per call.  Holds references to every buffer it
    was recorded with: write new tokens into `x` in place and call launch()."""

    def __init__(self, x: torch.Tensor, w_gate: torch.Tensor, w13: torch.Tensor,
                 w2: torch.Tensor, top_k: int, scales: Optional[Sequence[torch.Tensor]] = None,
                 out: Optional[torch.Tensor] = None, *, block_m: int = 0,
                 workspace: Optional[torch.Tensor] = None, act_quant: Optional[str] = None,
                 schedule: str = "auto"):
        self._h = None
        T, d, E, I = _shapes(x, w_gate, w13, w2)
        if out is not None:
            _check_out(out, x)
        dev = _dev(x, w_gate, w13, w2, out)
        desc = make_desc(T, d, E, I, _act_code(x), _w_code(w13), block_m, act_quant, schedule)
        self._sc = _scales(w13, scales)
        s = torch.cuda.current_stream(dev)
        own_out = out is None
        if own_out:
            out = _alloc((T, d), x.dtype, dev, s)
        nbytes = moe_workspace_bytes(desc, top_k, True)
        ws = _workspace(nbytes, dev, workspace, s)
        # the graph keeps these addresses: keep the tensors alive with it
        self._keep = (x, w_gate, w13, w2, tuple(scales) if scales is not None else None, ws)
        # tensors allocated here, which a replay on another stream must keep
        # from being reused before it has run
        self._owned = ([ws] if workspace is None else []) + ([out] if own_out else [])
        self.x, self.out, self.device = x, out, dev
        h = ctypes.c_void_p()
        _check("moe_graph_create", lib().moe_graph_create(
            ctypes.byref(desc), _ptr(x), _ptr(w_gate), _ptr(w13), _ptr(w2), int(top_k),
            ctypes.byref(self._sc) if self._sc is not None else None, _ptr(out), _ptr(ws), nbytes,
            ctypes.byref(h)))
        self._h = h

    def launch(self, stream=None) -> torch.Tensor:
        if self._h is None:
            raise RuntimeError("graph already destroyed")
        s = _launch_stream(self.device, stream)
        _check("moe_graph_launch", lib().moe_graph_launch(self._h, ctypes.c_void_p(s.cuda_stream)))
        if s != torch.cuda.current_stream(self.device):
            for t in self._owned:
                t.record_stream(s)
        return self.out

    def close(self) -> None:
        if self._h is not None:
            h, self._h = self._h, None
            _check("moe_graph_destroy", lib().moe_graph_destroy(h))

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def moe_expert_ffn(x: torch.Tensor, w13: torch.Tensor, w2: torch.Tensor, top_k: int,
                   topk_w: torch.Tensor, sorted_ids: torch.Tensor, block_expert: torch.Tensor,
                   num_padded: torch.Tensor, scales: Optional[Sequence[torch.Tensor]] = None,
                   out: Optional[torch.Tensor] = None, *, block_m: int = 0,
                   workspace: Optional[torch.Tensor] = None, stream=None,
                   act_quant: Optional[str] = None, schedule: str = "auto") -> torch.Tensor:
    """Expert networks + combine for a given routing (layout from moe_align
    with the same block_m and act_quant)."""
    T, d, E, I = _shapes(x, None, w13, w2)
    if out is not None:
        _check_out(out, x)
    desc = make_desc(T, d, E, I, _act_code(x), _w_code(w13), block_m, act_quant, schedule)
    B, cap = moe_align_capacity(desc, top_k)
    _check_routing(T, int(top_k), topk_w, sorted_ids, block_expert, num_padded, cap, B)
    dev = _dev(x, w13, w2, topk_w, sorted_ids, block_expert, num_padded, out)
    sc = _scales(w13, scales)
    s = _launch_stream(dev, stream)
    if out is None:
        out = _alloc((T, d), x.dtype, dev, s)
    nbytes = moe_workspace_bytes(desc, top_k, False)
    ws = _workspace(nbytes, dev, workspace, s)
    st = lib().moe_expert_ffn(ctypes.byref(desc), _ptr(x), _ptr(w13), _ptr(w2), int(top_k),
                              ctypes.byref(sc) if sc is not None else None, _ptr(topk_w),
                              _ptr(sorted_ids), _ptr(block_expert), _ptr(num_padded), _ptr(out),
                              _ptr(ws), nbytes, ctypes.c_void_p(s.cuda_stream))
    _check("moe_expert_ffn", st)
    return out


MOE_TIMING_ALL = (1 << MOE_KERNEL_COUNT) - 1
KERNEL_KINDS = {"route_logits": 0, "route_topk": 1, "align": 2, "ffn13": 3, "ffn2": 4, "combine": 5,
                "quant_x": 6, "ffn_fused": 7}


def moe_timing_enable(kinds=True) -> None:
    """Time the given kernel kinds: True = all, False/None = none, or an
    iterable of kind names ("ffn13", ...)."""
    if kinds is True:
        mask = MOE_TIMING_ALL
    elif not kinds:
        mask = 0
    else:
        mask = 0
        for k in kinds:
            mask |= 1 << KERNEL_KINDS[k]
    _check("moe_timing_enable", lib().moe_timing_enable(mask))


def moe_timing_collect(reset: bool = True) -> dict:
    """{kernel name: (total ms, launches)} for the kernels timed so far."""
    ms = (ctypes.c_double * MOE_KERNEL_COUNT)()
    n = (ctypes.c_int64 * MOE_KERNEL_COUNT)()
    _check("moe_timing_collect", lib().moe_timing_collect(ms, n, int(bool(reset))))
    return {moe_kernel_name(i): (ms[i], n[i]) for i in range(MOE_KERNEL_COUNT)}


def moe_kernel_name(kind: int) -> str:
    return lib().moe_kernel_name(int(kind)).decode()
