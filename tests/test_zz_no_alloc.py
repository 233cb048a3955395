"""moe_forward_noalloc: the layer with the library's static workspace
(one device array per GPU, no allocation in the call), checked against
moe_forward with a caller workspace on the same inputs: the same kernels
and launch plan, so the outputs must be equal bit for bit.  Two calls in a
row, the second with a smaller batch, so the second runs on a workspace the
first one left full of its own values."""

import dataclasses
import sys

import pytest
import torch

from mixture_experts_moe_amd import binding as B
from mixture_experts_moe_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


def note(msg):
    print(msg, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def loaded():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    B.lib()


def _pair(inp, bm=0):
    sc = (inp.s13, inp.s2) if inp.w == "e4m3fn" else None
    ref = B.moe_forward(inp.x, inp.w_gate, inp.w13, inp.w2, inp.top_k, sc, block_m=bm)
    out = torch.full_like(inp.x, float("nan"))
    B.moe_forward_noalloc(inp.x, inp.w_gate, inp.w13, inp.w2, inp.top_k, out, sc, block_m=bm)
    torch.cuda.synchronize()
    return out, ref


# workload, overrides, the two batch sizes (second smaller), block_m
CASES = [
    ("decode_bf16", dict(), (64, 8), 0),                       # the decode shape, LDS streaming
    ("decode_bf16", dict(), (8, 1), 0),                        # routing + regrouping in one kernel
    ("decode_bf16", dict(d=512, I=512, x_std=1.0), (300, 200), 128),   # 128-token GEMM, queue
    ("fp8", dict(d=512, I=512, E=16, k=4), (64, 9), 0),        # e4m3fn weights
    ("tiny_fp32", dict(), (37, 16), 0),
]


@pytest.mark.parametrize("wl,over,Ts,bm", CASES, ids=[f"{c[0]}-{c[2]}" for c in CASES])
def test_noalloc_equals_forward_twice_smaller_second(wl, over, Ts, bm):
    base = synth.make_inputs(wl, T=Ts[0], device=DEV, **over)
    cfg = synth.WORKLOADS[wl]
    for T in Ts:
        note(f"noalloc {wl} T={T} B={bm} {over}")
        x = synth.make_x(T, base.d, base.act, over.get("x_std", cfg["x_std"]), T, DEV)
        inp = dataclasses.replace(base, x=x)
        out, ref = _pair(inp, bm)
        assert torch.equal(out, ref), f"T={T}: noalloc output differs from moe_forward"


def test_noalloc_rejects_a_layer_beyond_its_array():
    # 20000 tokens at d = I = 512, top-2: h and the W2 partials need about
    # 120 MiB of workspace, more than the 64 MiB array
    inp = synth.make_inputs("decode_bf16", T=20000, device=DEV, d=512, I=512, x_std=1.0)
    desc = B.make_desc(inp.T, inp.d, inp.E, inp.I, B.MOE_DTYPE_BF16, B.MOE_DTYPE_BF16)
    assert B.moe_workspace_bytes(desc, inp.top_k, True) > B.MOE_NOALLOC_WORKSPACE_BYTES
    out = torch.full_like(inp.x, float("nan"))
    with pytest.raises(B.MoEError) as ei:
        B.moe_forward_noalloc(inp.x, inp.w_gate, inp.w13, inp.w2, inp.top_k, out)
    assert ei.value.status == B.MOE_ERR_NOALLOC_SIZE
    torch.cuda.synchronize()
    assert torch.isnan(out.float()).all(), "a rejected call must enqueue nothing"
