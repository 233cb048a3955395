"""Host-side argument checks of the Python binding: mismatched dtypes and
shapes raise before any device access or launch.  The tensors live on
torch's "meta" device (shapes and dtypes only, no memory), so nothing here
needs a GPU; the binding checks metadata before it looks at devices."""

import os

import pytest
import torch

from mixture_experts_moe_amd import binding as B

META = "meta"


@pytest.fixture(scope="module", autouse=True)
def lib():
    if not os.path.exists(B._LIB_PATH):
        from mixture_experts_moe_amd import build
        build.build()
    return B.lib()


def layer(T=4, d=128, E=4, I=128, w=torch.bfloat16, w2=None):
    x = torch.empty(T, d, dtype=torch.bfloat16, device=META)
    wg = torch.empty(E, d, dtype=torch.float32, device=META)
    w13 = torch.empty(E, 2 * I, d, dtype=w, device=META)
    w2t = torch.empty(E, d, I, dtype=w2 or w, device=META)
    return x, wg, w13, w2t


@pytest.mark.parametrize("w13_dtype,w2_dtype", [
    (torch.bfloat16, torch.uint8),           # W2 would be read as bf16: twice its size
    (torch.uint8, torch.bfloat16),
    (torch.bfloat16, torch.float32),
    (torch.float32, torch.bfloat16),
])
def test_weight_formats_must_agree(w13_dtype, w2_dtype):
    x, wg, w13, w2 = layer(w=w13_dtype, w2=w2_dtype)
    with pytest.raises(TypeError, match="one weight format"):
        B.moe_forward(x, wg, w13, w2, 2)
    with pytest.raises(TypeError, match="one weight format"):
        B.MoeGraph(x, wg, w13, w2, 2)
    ids = torch.empty(x.shape[0], 2, dtype=torch.float32, device=META)
    i32 = torch.empty(64, dtype=torch.int32, device=META)
    with pytest.raises(TypeError, match="one weight format"):
        B.moe_expert_ffn(x, w13, w2, 2, ids, i32, i32, i32)


@pytest.mark.parametrize("shape,dtype", [((4, 64), torch.bfloat16), ((3, 128), torch.bfloat16),
                                         ((4, 128), torch.float32)])
def test_out_must_match_x(shape, dtype):
    x, wg, w13, w2 = layer()
    out = torch.empty(shape, dtype=dtype, device=META)
    with pytest.raises(ValueError, match="out must match x"):
        B.moe_forward(x, wg, w13, w2, 2, out=out)
    with pytest.raises(ValueError, match="out must match x"):
        B.MoeGraph(x, wg, w13, w2, 2, out=out)
    tw = torch.empty(4, 2, dtype=torch.float32, device=META)
    i32 = torch.empty(1024, dtype=torch.int32, device=META)
    with pytest.raises(ValueError, match="out must match x"):
        B.moe_expert_ffn(x, w13, w2, 2, tw, i32, i32, i32, out=out)


def test_expert_ffn_checks_routing_tensors():
    x, wg, w13, w2 = layer()
    T, k = x.shape[0], 2
    _, cap = B.moe_align_capacity(B.make_desc(T, 128, 4, 128, B.MOE_DTYPE_BF16,
                                              B.MOE_DTYPE_BF16), k)
    good_w = torch.empty(T, k, dtype=torch.float32, device=META)
    good_i = torch.empty(cap, dtype=torch.int32, device=META)
    one = torch.empty(1, dtype=torch.int32, device=META)
    bad = [
        (dict(topk_w=torch.empty(T, k, dtype=torch.bfloat16, device=META)), ValueError),
        (dict(topk_w=torch.empty(T, k + 1, dtype=torch.float32, device=META)), ValueError),
        (dict(topk_w=torch.empty(T + 1, k, dtype=torch.float32, device=META)), ValueError),
        (dict(sorted_ids=torch.empty(cap, dtype=torch.int64, device=META)), TypeError),
        (dict(block_expert=torch.empty(cap, dtype=torch.int16, device=META)), TypeError),
        (dict(num_padded=torch.empty(1, dtype=torch.float32, device=META)), TypeError),
        (dict(sorted_ids=torch.empty(cap - 1, dtype=torch.int32, device=META)), ValueError),
        (dict(num_padded=torch.empty(0, dtype=torch.int32, device=META)), ValueError),
    ]
    for over, exc in bad:
        args = dict(topk_w=good_w, sorted_ids=good_i, block_expert=good_i, num_padded=one)
        args.update(over)
        with pytest.raises(exc):
            B.moe_expert_ffn(x, w13, w2, k, args["topk_w"], args["sorted_ids"],
                             args["block_expert"], args["num_padded"])


def test_x_must_be_two_dimensional():
    x, wg, w13, w2 = layer()
    with pytest.raises(ValueError, match=r"x must be \[T, d\]"):
        B.moe_forward(x.reshape(2, 2, 128), wg, w13, w2, 2)


def test_checks_pass_then_the_device_check_refuses_meta_tensors():
    # consistent metadata gets as far as the device check (a meta tensor is
    # not on the GPU), i.e. the checks above are the ones that fired
    x, wg, w13, w2 = layer()
    with pytest.raises(ValueError, match="on the GPU"):
        B.moe_forward(x, wg, w13, w2, 2)
