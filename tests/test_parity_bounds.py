"""The derived parity bounds of tests/parity_utils.py, exercised on the CPU.

A stand-in for the GPU result is built from the oracle's own intermediates
with the GPU path's rounding points (h stored as bf16 and the output rounded
to bf16, both to nearest even; fp32 layers unrounded), then fed to
compare_layer: it must pass, and planted mistakes of the kind the stated
Frobenius bounds could hide must fail.  Everything runs on CPU tensors."""

import numpy as np
import pytest
import torch

import parity_utils as PU
from mixture_experts_moe_amd import synth


def _bf16(a: np.ndarray) -> np.ndarray:
    return torch.from_numpy(a).to(torch.float32).to(torch.bfloat16).to(torch.float64).numpy()


def emulate(inp, round_h=True):
    """(out as the GPU would store it, routing ids) from the oracle's
    per-slot h, with h and out rounded where the GPU rounds them."""
    store = {}

    def hook(p):
        h = p["h_used"]
        if round_h and inp.act == "bf16" and inp.act_quant is None:
            h = _bf16(h)
        store[int(p["e"])] = (p["slots"], p["gates"][:, None] * (h @ p["w2"].T))

    ref = PU.oracle_layer(inp, expert_hook=hook)
    T, k, d = inp.T, inp.top_k, inp.d
    y = np.zeros((T * k, d))
    for fs, ys in store.values():
        y[fs] = ys
    out = y.reshape(T, k, d).sum(axis=1)
    t = torch.from_numpy(out)
    t = t.to(torch.bfloat16) if inp.act == "bf16" else t.to(torch.float32)
    return t, torch.from_numpy(ref["ids"]).to(torch.int32)


CASES = [
    ("tiny_fp32", dict(), 16),
    ("decode_bf16", dict(d=512, I=448, x_std=1.0), 12),
    ("decode_bf16", dict(d=256, I=128, E=8, k=8, x_std=1.0), 6),
    ("fp8", dict(d=256, I=192, E=16, k=4), 9),
    ("fp8", dict(d=256, I=256, E=4, k=2, act_quant="mx_e4m3"), 7),
]


@pytest.mark.parametrize("wl,over,T", CASES, ids=[f"{c[0]}-{c[2]}" for c in CASES])
def test_emulated_gpu_rounding_passes(wl, over, T):
    inp = synth.make_inputs(wl, T=T, **over)
    out, ids = emulate(inp)
    r = PU.compare_layer(inp, out, ids)
    print(wl, T, {k: v for k, v in r.items() if k != "ids"})


@pytest.mark.parametrize("wl,over,T", CASES[1:4], ids=[f"{c[0]}-{c[2]}" for c in CASES[1:4]])
def test_ten_percent_on_one_channel_tile_fails(wl, over, T):
    """The case the single Frobenius ratio missed: 10% off on 16 channels of
    one token moves the layer's relative error by about 1e-3."""
    inp = synth.make_inputs(wl, T=T, **over)
    out, ids = emulate(inp)
    bad = out.clone()
    bad[T // 2, 32:48] = (bad[T // 2, 32:48].double() * 1.1).to(bad.dtype)
    with pytest.raises(AssertionError, match="element bound"):
        PU.compare_layer(inp, bad, ids)


def test_dropped_slot_fails():
    inp = synth.make_inputs("decode_bf16", T=10, d=256, I=128, E=8, k=4, x_std=1.0)
    store = {}
    ref = PU.oracle_layer(inp, expert_hook=lambda p: None)
    # the output without the token's last slot
    y = ref["y_slot"].reshape(inp.T, inp.top_k, inp.d)
    out = torch.from_numpy(y[:, :-1].sum(axis=1)).to(torch.bfloat16)
    with pytest.raises(AssertionError):
        PU.compare_layer(inp, out, torch.from_numpy(ref["ids"]).to(torch.int32))


def test_unrounded_and_fp32_h_pass_too():
    # h kept in fp32 (a tighter GPU) is still inside the bf16 bounds
    inp = synth.make_inputs("decode_bf16", T=8, d=256, I=256, x_std=1.0)
    out, ids = emulate(inp, round_h=False)
    PU.compare_layer(inp, out, ids)


def test_w8a8_flip_accounting():
    """In the W8A8 mode the oracle's h values that sit within the GPU's fp32
    error of an e4m3fn rounding boundary are found and bounded: a forced flip
    of one such value by one code step stays inside the bound."""
    inp = synth.make_inputs("fp8", T=20, d=256, I=256, E=4, k=2, act_quant="mx_e4m3")
    out, ids = emulate(inp)
    r = PU.compare_layer(inp, out, ids)
    assert 0 <= r["flips"] < r["h_values"]


def test_flip_dev_is_zero_away_from_boundaries():
    # exact codes at block scales 2^-8 and 2^-13 (384 * scale), maxima far
    # from a power of two: nothing can flip
    h = np.array([[1.5] * 32, [3.0 * 2 ** -6] * 32])
    eps = np.full_like(h, 1e-9)
    assert not PU._mx_flip_dev(h, eps).any()
    # a value on a midpoint between two codes (1.0625 between 1 and 1.125 at
    # scale 2^0, block maximum 300) can flip by one step; its neighbours not
    h2 = np.array([[300.0] + [1.0625] + [1.0] * 30])
    dev = PU._mx_flip_dev(h2, np.full_like(h2, 1e-6))
    assert dev[0, 1] == pytest.approx(0.125) and dev[0, 2] == 0.0
    # a block maximum at a power of two may quantise with either exponent:
    # every value of the block is then bounded loosely, never by zero
    h3 = np.array([[256.0] + [1.0] * 31])
    assert (PU._mx_flip_dev(h3, np.full_like(h3, 1e-6)) > 0).all()


def test_covering_tokens_hit_every_block():
    rng = np.random.default_rng(3)
    T, E, k, B = 500, 16, 4, 32
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    toks = PU.covering_tokens(ids, E, B, extra=0)
    import oracle
    al = oracle.align(ids, E, B)
    chosen_slots = set((t * k + j) for t in toks for j in range(k))
    srt = al["sorted_ids"]
    for b in range(al["num_padded"] // B):
        blk = srt[b * B:(b + 1) * B]
        real = blk[blk < T * k]
        assert int(real[0]) in chosen_slots and int(real[-1]) in chosen_slots
