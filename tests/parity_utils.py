"""Shared helpers of the GPU parity tests (test code only)."""

import dataclasses

import numpy as np
import torch

import oracle
from mixture_experts_moe_amd import synth

TIE_GAP = 1e-4          # tokens whose k-th / (k+1)-th logit gap is below this are excluded
TOL = {"f32": 1e-5, "bf16": 2e-2, "e4m3fn": 6e-2}
# Tighter bound derived from where the kernels round: the GPU computes in
# fp32 and rounds only h and out to bf16 (relative 2^-9 each, to nearest
# even), and e4m3fn weights are widened to bf16 exactly, so against the fp64
# oracle fed the same bytes the relative Frobenius error is ~2e-3 for bf16 and
# e4m3fn weights alike.  5e-3 catches systematic errors (a wrong dequantised
# code, a dropped scale) that the looser bound above could hide.
DERIVED_TOL = {"f32": 1e-5, "bf16": 5e-3, "e4m3fn": 5e-3}
# The W8A8 mode adds one more rounding point: h is quantised to e4m3fn from
# fp32 on the GPU and from fp64 in the oracle, so a value within fp32 error of
# a rounding midpoint takes the neighbouring code (one step, 6-12% of that
# value).  Over many slots those flips are rare and average out (measured
# 1.7-2.3e-3 at 37+ tokens), but with a handful of slots one flip moves the
# relative error by a few 1e-3 (4.3e-3 at T = 2): the mode's derived bound is
# 1e-2, still far below anything a wrong block exponent (a factor of 2) or a
# lost block would give.
DERIVED_TOL_W8A8 = 1e-2


def rel_fro(got: np.ndarray, ref: np.ndarray) -> float:
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / den) if den > 0 else float(np.linalg.norm(got))


def near_ties(logits64: np.ndarray, k: int, gap: float = TIE_GAP) -> np.ndarray:
    """Boolean mask of tokens whose k-th and (k+1)-th largest logits are
    closer than `gap` (nothing is excluded when k = E)."""
    T, E = logits64.shape
    if k >= E or T == 0:
        return np.zeros(T, dtype=bool)
    s = -np.sort(-logits64, axis=1)
    return (s[:, k - 1] - s[:, k]) < gap


def subset(inp: synth.MoEInputs, tokens) -> synth.MoEInputs:
    idx = torch.as_tensor(np.asarray(tokens, dtype=np.int64), device=inp.x.device)
    return dataclasses.replace(inp, x=inp.x.index_select(0, idx).contiguous())


def with_x(inp: synth.MoEInputs, x: torch.Tensor) -> synth.MoEInputs:
    return dataclasses.replace(inp, x=x)


def oracle_layer(inp: synth.MoEInputs, block_m: int = 16, logits=None) -> dict:
    kw = synth.to_oracle(inp)
    return oracle.moe_forward(**kw, block_m=block_m, logits=logits)


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to(torch.float64).cpu().numpy()


def compare_layer(inp: synth.MoEInputs, out_gpu: torch.Tensor, gpu_ids: torch.Tensor,
                  tokens=None, tol=None) -> dict:
    """Oracle on `tokens` (all by default); check the GPU's routing on the
    tokens that are not near ties and the relative Frobenius error of the
    outputs over them.  Returns the measured numbers."""
    T = inp.T
    tokens = np.arange(T) if tokens is None else np.asarray(tokens)
    sub = subset(inp, tokens)
    ref = oracle_layer(sub)
    excl = near_ties(ref["logits"], inp.top_k)
    keep = ~excl
    ids_gpu = gpu_ids.cpu().numpy()[tokens]
    routed_same = np.array_equal(ids_gpu[keep], ref["ids"][keep])
    got = to_f64(out_gpu)[tokens]
    err = rel_fro(got[keep], ref["out"][keep])
    tol = TOL[inp.w] if tol is None else tol
    assert routed_same, "GPU routing differs from the oracle on a token that is not a near tie"
    assert np.all(np.isfinite(got)), "non-finite outputs"
    assert err <= tol, f"relative Frobenius error {err:.3e} > {tol:.1e}"
    derived = DERIVED_TOL_W8A8 if inp.act_quant else DERIVED_TOL[inp.w]
    assert err <= derived, (
        f"relative Frobenius error {err:.3e} above the bound derived from the kernels' rounding "
        f"({derived:.1e})")
    return {"rel_err": err, "excluded": int(excl.sum()), "compared": int(keep.sum())}
