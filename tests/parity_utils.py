"""Shared helpers of the GPU parity tests (test code only).

Layer outputs are judged three ways against the fp64 oracle, on the tokens
that are not near routing ties:

1. the stated relative Frobenius bound of the weight format (fp32 1e-5,
   bf16 2e-2, e4m3fn 6e-2) over all compared tokens;
2. bounds derived from where the HIP kernels round, computed for these very
   inputs from the oracle's own intermediates (``LayerBounds``):
     - every element:  |got - ref| <= u_out |ref| + Z * sqrt(V) + D
     - every token:    ||got_t - ref_t|| <= TOKEN_Z * sqrt(sum_c var) + ||D_t||
     - all compared:   ||got - ref||_F <= GLOBAL_Z * sqrt(sum var) + ||D||_F
   with the terms below;
3. the GPU's routing equals the oracle's on every compared token.

Error model of the GPU path (what the kernels do, checked against the
sources): products of bf16 / e4m3fn-widened-to-bf16 / fp32 operands are exact
in fp32 and summed in fp32; the router's logits are fp32 sums; the gates are
an fp32 softmax; h = SiLU(g) * u is formed in fp32 and stored as bf16 (fp32
for fp32 layers, e4m3fn codes in the W8A8 mode); W2 sums in fp32; the k slot
outputs are added in fp32 and the result rounded once to the output format,
to nearest even.  With u the unit roundoff of a format (bf16 2^-8: 8
significant bits; fp32 2^-24):

  h rounding      each stored h_i = h_i (1 + delta_i), |delta_i| <= u_h, the
                  delta_i independent with mean 0.  The resulting error of an
                  output element is sum_i a_i delta_i with a_i = gate W2[c,i]
                  h_i, so (Hoeffding) P(|err| > Z u_h sqrt(S)) <= 2 exp(-Z^2/2)
                  with S = sum_i a_i^2; for Z = 7 that is 4.6e-11 per element.
                  Its variance is at most u_h^2 S / 3 (an error uniform within
                  half a unit in the last place).
  fp32 sums       a sum of n products carries an error of standard deviation
                  at most sqrt(n) u32 sqrt(sum of squared products) (recursive
                  summation; blocked MFMA sums do better).  For W13 this
                  perturbs g and u before the SiLU product, dh_i = |SiLU'(g)
                  u| dg + |SiLU(g)| du + SILU_ULPS u32 |h| (the SiLU
                  evaluation, exp and reciprocal included); its effect on an
                  output has variance sum_i (gate W2[c,i])^2 dh_i^2.  For W2 it
                  is I u32^2 S.
  gates           the logits' fp32 sums move each selected logit by dl (as
                  above, over d products); a softmax gate then moves by at
                  most 2 Z max dl relative, plus SILU_ULPS u32 for its own
                  evaluation: a deterministic term times sum_j |y_j|.
  combine         k fp32 additions: at most (k + 8) u32 sum_j |y_j| (the gate
                  and fp8 scale products included).
  out rounding    u_out |ref| (u_out = 2^-8 for bf16 outputs, 2^-24 for fp32).
  W8A8 mode       the scaled fp8 MFMA (v_mfma_scale_f32_16x16x128_f8f6f4)
                  does not sum its 128 products in fp32: it aligns products
                  to a larger one and drops low bits.  Model (measured on the
                  device; tests/test_gpu_numerics.py checks it every run):
                  with E the exponent of the step's largest product, a
                  product whose exponent is at least E - 6 loses nothing and
                  a smaller one less than min(|p|, 2^(E - 13)).  So a sum
                  over K carries Hoeffding scale sqrt(sum of those squared
                  losses), computed per product for small weights and
                  otherwise bounded by 2^-13 sqrt(128 sum_steps max |p|^2)
                  (with max|x| max|w| per 128-K step, or the sum of squared
                  products).  x is quantised
                  identically on both sides (bit-exact, tested separately),
                  so the only h difference is a code flip: a value whose
                  deviation Z dh_i (W13's MFMA sums, then SiLU) can carry it
                  across an e4m3fn rounding boundary, or a 32-value block
                  whose maximum can cross a power of two (its exponent may
                  then differ).  Every such value is found from the oracle's
                  h; its largest possible difference dev_i enters as a
                  bounded, zero-mean term: Z sqrt(sum_i (gate W2[c,i]
                  dev_i)^2).  All other values quantise to the same code on
                  both sides.  W2's own MFMA sums add the same kind of term
                  over I.

Near-tie tokens (k-th / (k+1)-th logit gap below 1e-4 in the oracle's
logits) are excluded, as the stated rule says: their routing may
legitimately differ.
"""

import dataclasses
import math
import os
import threading

import numpy as np
import torch

import oracle
from oracle import moe_oracle as _om
from mixture_experts_moe_amd import synth

TIE_GAP = 1e-4          # tokens whose k-th / (k+1)-th logit gap is below this are excluded
TOL = {"f32": 1e-5, "bf16": 2e-2, "e4m3fn": 6e-2}

U32 = 2.0 ** -24        # fp32 unit roundoff
U_BF16 = 2.0 ** -8      # bf16 unit roundoff (8 significant bits, round to nearest even)
Z = 7.0                 # element bound: 2 exp(-Z^2 / 2) = 4.6e-11 per element
TOKEN_Z = 3.0           # per-token norm against its root-mean-square bound
GLOBAL_Z = 2.0          # whole comparison (many more independent terms)
SILU_ULPS = 8           # fp32 ulps of |h| for SiLU(g) * u and its scale products
FP8_MFMA_GROUP = 128    # the scaled fp8 MFMA's K step (products aligned within it)
FP8_MFMA_BITS = 13      # bits kept below the step's largest product
EXACT_MFMA_ELEMS = 1 << 24   # weight matrices up to this size get the per-product bound


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


ORACLE_WORKERS = min(16, len(os.sched_getaffinity(0)))


def oracle_layer(inp: synth.MoEInputs, block_m: int = 16, logits=None, expert_hook=None) -> dict:
    """The oracle on these inputs, its experts spread over ORACLE_WORKERS
    threads (single-threaded BLAS inside them: the per-expert products are
    skinny, and nested thread pools would oversubscribe the cores)."""
    import threadpoolctl
    kw = synth.to_oracle(inp)
    with threadpoolctl.threadpool_limits(1):
        return oracle.moe_forward(**kw, block_m=block_m, logits=logits, expert_hook=expert_hook,
                                  workers=ORACLE_WORKERS)


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to(torch.float64).cpu().numpy()


# ---------------------------------------------------------------- derived bounds

def _e4m3_value(y: np.ndarray) -> np.ndarray:
    """Value of the e4m3fn code nearest to y (|y| clamped to 448 first),
    ties to even: the oracle's own rounding."""
    c = _om._e4m3fn_nearest(np.clip(y, -_om.E4M3_MAX, _om.E4M3_MAX))
    return oracle.decode_e4m3fn(c)


def _mx_flip_dev(h: np.ndarray, eps: np.ndarray, scale: np.ndarray = None):
    """Largest possible |q_gpu - q_oracle| per value when the GPU's h may
    differ from the oracle's h by up to eps (rows of 32-value blocks,
    quantised as mx_quantize does); 0 where both must give the same code.
    With `scale` (the Hoeffding scale of the GPU's deviation from h) also
    returns a bound on each value's flip probability: 2 exp(-D^2 / (2
    scale^2)) for a value at distance D from its nearest rounding boundary,
    1 in blocks whose exponent may differ."""
    n, I = h.shape
    B = _om.MX_BLOCK
    hb = h.reshape(n, I // B, B)
    eb = eps.reshape(n, I // B, B)
    ab = np.abs(hb)
    amax_lo = np.max(np.maximum(ab - eb, 0.0), axis=2)
    amax_hi = np.max(ab + eb, axis=2)

    def expo(a):
        out = np.zeros(a.shape, dtype=np.int64)
        nz = a > 0
        _, e = np.frexp(a[nz])
        out[nz] = np.clip(e - 1 - _om.E4M3_EMAX, _om.E8M0_EMIN, _om.E8M0_EMAX)
        return out

    e_lo, e_hi = expo(amax_lo), expo(amax_hi)
    zero_lo = amax_lo == 0
    fixed = (e_lo == e_hi) & ~(zero_lo & (amax_hi > 0))
    X = np.ldexp(1.0, e_hi)[:, :, None]
    # blocks with one exponent: a value can only flip if h - eps and h + eps
    # round to different codes; the difference is then at most the span
    q_lo = _e4m3_value((hb - eb) / X) * X
    q_hi = _e4m3_value((hb + eb) / X) * X
    span = np.abs(q_hi - q_lo)
    dev = np.where(fixed[:, :, None], span, 0.0)
    # blocks whose exponent may differ: each side is within its rounding (or
    # clamp) error of its own h: <= 2^-3 |v| + 2^-10 X
    X_lo = np.ldexp(1.0, e_lo)[:, :, None]
    loose = (2.0 ** -3) * (2 * ab + eb) + eb + (2.0 ** -10) * (X + X_lo)
    dev = np.where(fixed[:, :, None], dev, loose).reshape(n, I)
    if scale is None:
        return dev
    # distance of |h| / X to the nearest rounding boundary (the midpoints
    # between neighbouring e4m3fn values), for the flip probability
    pos = _om._E4M3_POS
    mids = (pos[1:] + pos[:-1]) / 2
    y = np.minimum(ab / X, _om.E4M3_MAX)
    j = np.clip(np.searchsorted(mids, y), 1, mids.size - 1)
    dist = np.minimum(np.abs(y - mids[j - 1]), np.abs(mids[j] - y)) * X
    sc = np.maximum(scale.reshape(n, I // B, B), 1e-300)
    prob = np.minimum(1.0, 2.0 * np.exp(-dist * dist / (2 * sc * sc)))
    prob = np.where(fixed[:, :, None], prob, 1.0).reshape(n, I)
    return dev, np.where(dev > 0, prob, 0.0)


class LayerBounds:
    """Collects, through the oracle's expert hook, the per-slot terms of the
    derived bounds (see the module docstring), then evaluates them for the
    oracle's output."""

    def __init__(self, inp: synth.MoEInputs, T: int):
        self.k, self.d, self.I = inp.top_k, inp.d, inp.I
        self.mx = inp.act_quant is not None
        self.u_h = 0.0 if self.mx else (U32 if inp.act == "f32" else U_BF16)
        self.u_out = U32 if inp.act == "f32" else U_BF16
        A = T * self.k
        self.S = np.zeros((A, self.d))      # sum_i (gate W2 h_used)^2
        self.R = np.zeros((A, self.d))      # further Hoeffding scale^2 (accumulation, flips)
        self.Rv = np.zeros((A, self.d))     # their variance where it is smaller (flips)
        self.flips = 0
        self.values = 0
        self._lock = threading.Lock()   # the oracle may run experts in threads

    @staticmethod
    def _fp8_mfma_scale_exact(a: np.ndarray, w: np.ndarray) -> np.ndarray:
        """The same scale from every product of each 128-K step: one whose
        exponent is at least the step maximum's minus 6 loses nothing, a
        smaller one less than min(|p|, 2^(E_max - 13)).  The products here
        carry the weight row's fp32 scale, which can shift exponents by
        one, so both margins are widened by one (5 and 12)."""
        G = FP8_MFMA_GROUP
        n, K = a.shape
        out = np.empty((n, w.shape[0]), dtype=np.float64)
        wf = w.astype(np.float32)
        for r in range(n):
            p = np.abs(wf * a[r].astype(np.float32)[None, :]).reshape(w.shape[0], K // G, G)
            pmax = p.max(axis=2, keepdims=True)
            with np.errstate(divide="ignore"):
                e_k = np.floor(np.log2(np.where(p > 0, p, 1e-38)))
                e_g = np.floor(np.log2(np.where(pmax > 0, pmax, 1e-38)))
            c = np.where(e_k >= e_g - 5, 0.0, np.minimum(2 * p, np.exp2(e_g - 12)))
            out[r] = np.sqrt((c.astype(np.float64) ** 2).sum(axis=(1, 2)))
        return out

    @staticmethod
    def _fp8_mfma_scale(a: np.ndarray, w: np.ndarray, l2: np.ndarray) -> np.ndarray:
        """Hoeffding scale of the scaled fp8 MFMA's truncation over the K sum
        of a [n, K] . w [m, K]^T: every product's loss lies within
        2^-12 max_step |p| (one exponent of margin for the weight scale), so
        the scale is 2^-12 sqrt(128 sum_steps max_step |p|^2).  Two upper
        bounds of sum_steps max_step |p|^2 are at hand: sum_steps (max|a|
        max|w|)^2, and sum_k p_k^2 = l2^2 (a step's largest square is at
        most its sum of squares); the smaller is used."""
        G = FP8_MFMA_GROUP
        am = np.abs(a).reshape(a.shape[0], -1, G).max(axis=2).astype(np.float32)
        wm = np.abs(w).reshape(w.shape[0], -1, G).max(axis=2).astype(np.float32)
        mm = (am * am) @ (wm * wm).T
        return (2.0 ** (1 - FP8_MFMA_BITS)) * np.sqrt(G * np.minimum(mm, l2 * l2))

    def hook(self, p: dict) -> None:
        fs, x, w13, w2, gates = p["slots"], p["x"], p["w13"], p["w2"], p["gates"]
        g, u, h, hu = p["g"], p["u"], p["h"], p["h_used"]
        I, d = self.I, self.d
        W2sq = np.square(w2, dtype=np.float32)                     # [d, I]
        gsq = (gates * gates)[:, None]
        self.S[fs] = gsq * (np.square(hu, dtype=np.float32) @ W2sq.T)
        # W13's sums: deviation scale of g and u per (slot, channel)
        G = np.sqrt(np.square(x, dtype=np.float32) @ np.square(w13, dtype=np.float32).T)
        dg = math.sqrt(d) * U32 * G[:, :I] + U32 * np.abs(g)
        du = math.sqrt(d) * U32 * G[:, I:] + U32 * np.abs(u)
        if self.mx:
            if w13.size <= EXACT_MFMA_ELEMS:
                t13 = self._fp8_mfma_scale_exact(x, w13)
            else:
                t13 = self._fp8_mfma_scale(x, w13, G)
            dg = dg + t13[:, :I]
            du = du + t13[:, I:]
        with np.errstate(over="ignore"):
            sig = 1.0 / (1.0 + np.exp(-g))
        dsilu = np.abs(sig * (1.0 + g * (1.0 - sig)))
        dh = dsilu * np.abs(u) * dg + np.abs(g * sig) * du + SILU_ULPS * U32 * np.abs(h)
        if self.mx:
            dev, prob = _mx_flip_dev(h, Z * dh, dh)
            with self._lock:
                self.flips += int(np.count_nonzero(dev))
                self.values += dev.size
            l2 = np.sqrt(np.square(hu, dtype=np.float32) @ W2sq.T)    # [n, d]
            t2 = (self._fp8_mfma_scale_exact(hu, w2) if w2.size <= EXACT_MFMA_ELEMS
                  else self._fp8_mfma_scale(hu, w2, l2))                 # W2's sums [n, d]
            dev2 = np.square(dev, dtype=np.float32)
            self.R[fs] = gsq * (dev2 @ W2sq.T + t2 * t2)
            # a flip moves an output by at most |gate W2 dev| and happens
            # with probability at most prob: variance <= (gate W2 dev)^2 prob
            self.Rv[fs] = gsq * ((dev2 * prob.astype(np.float32)) @ W2sq.T + t2 * t2 / 3)
        else:
            self.R[fs] = gsq * (np.square(dh, dtype=np.float32) @ W2sq.T)
            self.Rv[fs] = self.R[fs] / 3

    def evaluate(self, ref: dict, x64: np.ndarray, w_gate: np.ndarray) -> dict:
        """Per-element bound `elem` [T, d], variance bound `var` [T, d] and
        deterministic part `det` [T, d] for the oracle result `ref`."""
        T, d = ref["out"].shape
        k, I = self.k, self.I
        out = ref["out"]
        S = self.S.reshape(T, k, d).sum(axis=1)
        R = self.R.reshape(T, k, d).sum(axis=1)
        Rv = self.Rv.reshape(T, k, d).sum(axis=1)
        abs_y = np.abs(ref["y_slot"]).reshape(T, k, d).sum(axis=1)
        # gates: the router's fp32 logits
        wg = np.asarray(w_gate, dtype=np.float64)
        L = np.sqrt((x64 * x64) @ (wg * wg).T)                      # [T, E]
        dl = math.sqrt(d) * U32 * L + U32 * np.abs(ref["logits"])
        dl_sel = np.take_along_axis(dl, ref["ids"].astype(np.int64), axis=1).max(axis=1)
        rel_gate = 2.0 * Z * dl_sel + SILU_ULPS * U32
        det = ((k + 8) * U32 + rel_gate[:, None]) * abs_y
        # Hoeffding scale^2 of the random terms: h rounding, the sums, flips
        rand_sq = (self.u_h ** 2) * S + R + I * U32 ** 2 * S
        var = (self.u_out * out) ** 2 / 3 + ((self.u_h ** 2) * S + I * U32 ** 2 * S) / 3 + Rv
        elem = self.u_out * np.abs(out) + Z * np.sqrt(rand_sq) + det
        return {"elem": elem, "var": var, "det": det}


def compare_layer(inp: synth.MoEInputs, out_gpu: torch.Tensor, gpu_ids: torch.Tensor,
                  tokens=None, tol=None) -> dict:
    """Oracle on `tokens` (all by default); check the GPU's routing on the
    tokens that are not near ties, then the stated relative Frobenius bound
    and the derived element, token and global bounds over them.  Returns the
    measured numbers."""
    T = inp.T
    tokens = np.arange(T) if tokens is None else np.asarray(tokens)
    sub = subset(inp, tokens)
    bounds = LayerBounds(inp, len(tokens))
    ref = oracle_layer(sub, expert_hook=bounds.hook)
    excl = near_ties(ref["logits"], inp.top_k)
    keep = ~excl
    ids_gpu = gpu_ids.cpu().numpy()[tokens]
    routed_same = np.array_equal(ids_gpu[keep], ref["ids"][keep])
    got = to_f64(out_gpu)[tokens]
    assert routed_same, "GPU routing differs from the oracle on a token that is not a near tie"
    assert np.all(np.isfinite(got)), "non-finite outputs"
    err = rel_fro(got[keep], ref["out"][keep])
    tol = TOL[inp.w] if tol is None else tol
    assert err <= tol, f"relative Frobenius error {err:.3e} > {tol:.1e}"

    x64 = (oracle.decode_bf16(synth.to_oracle(sub)["x"]) if inp.act == "bf16"
           else to_f64(sub.x))
    b = bounds.evaluate(ref, x64, inp.w_gate.detach().cpu().numpy())
    diff = np.abs(got - ref["out"])[keep]
    elem, var, det = b["elem"][keep], b["var"][keep], b["det"][keep]
    worst = diff / np.maximum(elem, 1e-300)
    i_worst = np.unravel_index(int(np.argmax(worst)), worst.shape) if worst.size else None
    assert worst.size == 0 or worst.max() <= 1.0, (
        f"element bound exceeded: |got - ref| = {diff[i_worst]:.3e} > {elem[i_worst]:.3e} at "
        f"compared token {int(i_worst[0])}, channel {int(i_worst[1])} (ratio {worst.max():.2f})")
    tok_err = np.linalg.norm(diff, axis=1)
    tok_bound = TOKEN_Z * np.sqrt(var.sum(axis=1)) + np.linalg.norm(det, axis=1)
    tok_ratio = tok_err / np.maximum(tok_bound, 1e-300)
    assert tok_ratio.size == 0 or tok_ratio.max() <= 1.0, (
        f"token bound exceeded at compared token {int(np.argmax(tok_ratio))}: "
        f"{tok_err.max():.3e} (ratio {tok_ratio.max():.2f})")
    glob_bound = GLOBAL_Z * math.sqrt(float(var.sum())) + float(np.linalg.norm(det))
    glob_err = float(np.linalg.norm(diff))
    assert glob_err <= glob_bound, (
        f"global bound exceeded: {glob_err:.3e} > {glob_bound:.3e}")
    den = float(np.linalg.norm(ref["out"][keep])) or 1.0
    return {"rel_err": err, "excluded": int(excl.sum()), "compared": int(keep.sum()),
            "elem_ratio": float(worst.max()) if worst.size else 0.0,
            "token_ratio": float(tok_ratio.max()) if tok_ratio.size else 0.0,
            "derived_rel": glob_bound / den,
            "flips": bounds.flips, "h_values": bounds.values,
            "ids": ref["ids"]}


# ---------------------------------------------------------------- token choice

def covering_tokens(ids: np.ndarray, E: int, block_m: int, extra: int = 8) -> np.ndarray:
    """Tokens whose slots include the first and the last real slot of every
    row block of the regrouped layout (so every touched expert and every
    expert's ragged tail block is checked), plus `extra` evenly spaced ones."""
    T, k = ids.shape
    A = T * k
    al = oracle.align(ids, E, block_m)
    srt = al["sorted_ids"]
    chosen = set()
    for b in range(al["num_padded"] // block_m):
        blk = srt[b * block_m:(b + 1) * block_m]
        real = blk[blk < A]
        if real.size:
            chosen.add(int(real[0]) // k)
            chosen.add(int(real[-1]) // k)
    chosen.update(int(t) for t in np.linspace(0, T - 1, min(extra, T)).astype(int))
    return np.array(sorted(chosen), dtype=np.int64)
