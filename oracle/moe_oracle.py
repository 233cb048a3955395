"""Plain CPU oracle of the fused Mixture-of-Experts layer.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the package
``mixture_experts_moe_amd``, its HIP kernels and its C-ABI library) may import,
call or link anything in this directory.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` use it.
It shares no code, table or helper with the GPU path; it reads raw input arrays
(bf16 as uint16 bit patterns, e4m3fn as uint8 bytes, fp32 as float32) and
decodes them itself.

Sources, cited by tag:
  [P1] "Amazon SageMaker AIにおけるMixture-of-Expertsカーネル最適化の深掘り"
       (Japanese summary page), sections "MoEモデルの原理と推論における課題"
       and "カスタムカーネルエンジニアリングの技術".
  [P2] "Az AWS új MoE-optimalizációkkal gyorsítja a SageMaker AI-t"
       (Hungarian news page), sections "A fused MoE a számítási folyamat több
       lépését egyesíti" (called §fused below) and "FP8 esetén a Triton backend
       bizonyult gyorsabbnak" (called §fp8).
  [P3] "Ingénierie de kernels Mixture-of-Experts sur Amazon SageMaker AI"
       (French summary page), first paragraph.

What the pages fix: the fused layer is token routing, regrouping of the data by
expert, the experts' computation and the aggregation of the expert results,
done as one batched operation instead of a sequential loop over experts
([P2] §fused, [P3] first paragraph, [P2] §fp8 for the aggregation).  The
fused operation must therefore give the result of that per-expert loop, and
this module IS that loop, written plainly.  The pages do not write out the
router, the expert network or the FP8 format; the readings taken here are:
  * router: logits = x . W_gate^T, the k experts with the largest logits (ties
    go to the lower expert index), gates = softmax over the selected logits
    (equal to the full softmax renormalised over the selection);
  * expert: SwiGLU, W13 = [W1 (gate, rows 0..I-1); W3 (up, rows I..2I-1)],
    y = W2 . (SiLU(W1 x) * (W3 x)), SiLU(z) = z / (1 + e^-z);
  * the gate weight scales the expert output; a token's output is the sum over
    its k slots in rank order;
  * FP8 weights are OCP e4m3fn bytes times an fp32 scale per output channel
    (or one per expert matrix); activations stay bf16, or, in the optional
    W8A8 mode ([P2] §fp8: FP8 scaling fused with the matrix product), are
    quantised to e4m3fn in blocks of 32 consecutive values of a row with one
    power-of-two scale per block (the OCP microscaling layout): x per token
    before W13, the SwiGLU output h per routing slot before W2;
  * regrouping: per-expert counts, each expert's group padded to a multiple of
    a block size B, groups laid out in expert order, inside a group the flat
    slot ids f = t*k + j ascending, pad slots hold the sentinel A = T*k.

Precision: every floating-point step is fp64 (inputs are decoded exactly).

Pins (tests that tie each function to something other than itself; all run
under ``-m "not gpu"``):
  decode_bf16 / decode_e4m3fn .. all 65536 / 256 codes against torch dtype
      casts, plus OCP e4m3fn landmark values (448, 2^-9, 2^-6, NaN codes);
  router_logits ................ one-hot activations pick W_gate columns;
      math.fsum brute force on non-square shapes;
  select_topk .................. Python ``sorted`` brute force, duplicated
      W_gate rows (ties), k = E, k = 1;
  gate_weights ................. closed form on logits ln(1..4), sum = 1,
      k = 1 gives exactly 1, scipy softmax over the selection;
  align ........................ brute force with Python lists, invariants
      (each slot once, multiples of B, sum of counts = A, sentinel), a
      hand-worked case;
  silu / expert_ffn ............ E = 1, k = 1 reduces to a dense SwiGLU MLP
      evaluated with torch.nn.functional.silu in fp64; scalar closed form;
  moe_forward .................. dense brute force (every expert on every
      token, masked by the selection); k = E with W_gate = 0 gives the mean
      of all experts; zero tokens; idle experts; the W8A8 mode against a
      dense brute force that quantises with torch's e4m3fn cast;
  mx_quantize .................. brute force over all 256 codes (nearest,
      ties to even); torch's float8_e4m3fn cast of the scaled, clamped
      values; representable values round-trip; the block maximum lands in
      [256, 512) before clamping; zero blocks; saturation; a block too small
      for the scale it asks for (the E8M0 range stops at 2^-127).
No function here is "parity unpinned".
"""

from __future__ import annotations

import math

import numpy as np

__all__ = [
    "decode_bf16",
    "decode_e4m3fn",
    "decode_weights",
    "router_logits",
    "select_topk",
    "gate_weights",
    "align_capacity",
    "align",
    "silu",
    "expert_ffn",
    "mx_quantize",
    "mx_dequantize",
    "moe_forward",
]


# --------------------------------------------------------------------------
# Exact decoding of the stored number formats
# --------------------------------------------------------------------------

def decode_bf16(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exactly.

    bf16 is the upper half of an IEEE binary32, so the value is the float32
    whose top 16 bits are the pattern and whose low 16 bits are zero.
    """
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def _e4m3fn_value(code: int) -> float:
    """One OCP e4m3fn code -> its value.

    OCP 8-bit floating point, E4M3 variant: 1 sign bit, 4 exponent bits with
    bias 7, 3 mantissa bits; exponent field 0 encodes subnormals m * 2^-9;
    there are no infinities and S.1111.111 is NaN, so the largest finite
    magnitude is 1.75 * 2^8 = 448.  (The pages only say "FP8" -- [P1]
    techniques section, [P2] §fp8; e4m3fn is the reading taken.)
    """
    sign = -1.0 if (code >> 7) & 1 else 1.0
    exp_field = (code >> 3) & 0xF
    mant = code & 0x7
    if exp_field == 0xF and mant == 0x7:
        return math.nan
    if exp_field == 0:
        return sign * mant * 2.0 ** -9
    return sign * (1.0 + mant / 8.0) * 2.0 ** (exp_field - 7)


_E4M3FN_TABLE = np.array([_e4m3fn_value(c) for c in range(256)], dtype=np.float64)


def decode_e4m3fn(codes) -> np.ndarray:
    """e4m3fn bytes (uint8) -> float64 values, exactly (NaN for the NaN codes)."""
    return _E4M3FN_TABLE[np.asarray(codes, dtype=np.uint8)]


def decode_weights(raw, fmt: str, scale=None) -> np.ndarray:
    """Decode one expert's weight matrix [rows, K] to float64.

    fmt: "f32" (float32 values), "bf16" (uint16 patterns) or "e4m3fn"
    (uint8 bytes).  For "e4m3fn", ``scale`` is either a vector of one fp32
    scale per row (per output channel) or a scalar (per tensor); the
    dequantised weight is code_value * scale, formed in fp64 where it is exact.
    """
    a = np.asarray(raw)
    if fmt == "f32":
        return a.astype(np.float32).astype(np.float64)
    if fmt == "bf16":
        return decode_bf16(a)
    if fmt == "e4m3fn":
        if scale is None:
            raise ValueError("e4m3fn weights need a scale")
        w = decode_e4m3fn(a)
        s = np.asarray(scale, dtype=np.float32).astype(np.float64)
        if s.ndim == 0:
            return w * s
        if s.shape != (w.shape[0],):
            raise ValueError(f"per-channel scale must have shape ({w.shape[0]},), got {s.shape}")
        return w * s[:, None]
    raise ValueError(f"unknown weight format {fmt!r}")


def _decode_act(x, fmt: str) -> np.ndarray:
    if fmt == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    if fmt == "bf16":
        return decode_bf16(x)
    raise ValueError(f"unknown activation format {fmt!r}")


# --------------------------------------------------------------------------
# Routing ([P2] §fused: "tokenek útválasztása"; [P3] first paragraph)
# --------------------------------------------------------------------------

def router_logits(x: np.ndarray, w_gate: np.ndarray) -> np.ndarray:
    """logits[t, e] = sum_i x[t, i] * W_gate[e, i], in fp64.

    x: [T, d] float64 values; w_gate: [E, d] (float32 values, used exactly).
    """
    x = np.asarray(x, dtype=np.float64)
    wg = np.asarray(w_gate, dtype=np.float32).astype(np.float64)
    return x @ wg.T


def select_topk(logits: np.ndarray, k: int) -> np.ndarray:
    """The k experts with the largest logits per token, in rank order.

    Rank order is descending logit; equal logits are ordered by ascending
    expert index, so the lower index wins a tie.  Returns int32 [T, k].
    (The pages name routing but not its rule; this is the reading taken.)
    """
    lg = np.asarray(logits, dtype=np.float64)
    T, E = lg.shape
    if not 1 <= k <= E:
        raise ValueError(f"top_k must be in [1, {E}], got {k}")
    expert_index = np.broadcast_to(np.arange(E), (T, E))
    # lexsort: the last key is the primary key.
    order = np.lexsort((expert_index, -lg), axis=-1)
    return order[:, :k].astype(np.int32)


def gate_weights(logits: np.ndarray, ids: np.ndarray) -> np.ndarray:
    """Softmax over the selected logits: w_j = e^(l_j - m) / sum_sel e^(l - m).

    m is the largest selected logit.  This equals the softmax over all E
    logits renormalised to sum to one over the k selected experts.
    """
    lg = np.asarray(logits, dtype=np.float64)
    sel = np.take_along_axis(lg, np.asarray(ids, dtype=np.int64), axis=1)
    if sel.shape[1] == 0:
        return sel
    m = sel.max(axis=1, keepdims=True)
    p = np.exp(sel - m)
    return p / p.sum(axis=1, keepdims=True)


# --------------------------------------------------------------------------
# Regrouping by expert ([P2] §fused: "az adatok átrendezése";
# [P3] first paragraph: "réordonnancement des données"; variable-size token
# groups: [P2] §fp8, [P3] third paragraph)
# --------------------------------------------------------------------------

def align_capacity(num_assignments: int, num_experts: int, block_m: int) -> int:
    """Upper bound on the padded row count, rounded up to a multiple of B.

    Each expert that receives at least one slot wastes at most B - 1 pad rows
    and at most min(E, A) experts receive a slot.
    """
    A, E, B = num_assignments, num_experts, block_m
    n = A + min(E, A) * (B - 1)
    return -(-n // B) * B


def align(ids: np.ndarray, num_experts: int, block_m: int) -> dict:
    """Regroup the T*k routing slots by expert, each group padded to B rows.

    Flat slot id f = t*k + j.  counts[e] = #slots routed to e.  Group e
    starts at off[e] = sum_{e'<e} ceil(counts[e']/B)*B and lists its slots in
    ascending f; the rest of the group is the sentinel A.  block_expert[b]
    is the expert owning rows [b*B, (b+1)*B); entries past the padded total
    are -1 and sorted_ids past it are A.
    """
    ids = np.asarray(ids, dtype=np.int64)
    T, k = ids.shape if ids.ndim == 2 else (0, 0)
    A = T * k
    E, B = int(num_experts), int(block_m)
    flat = ids.reshape(-1)
    counts = np.zeros(E, dtype=np.int64)
    for f in range(A):
        counts[flat[f]] += 1
    padded = -(-counts // B) * B
    off = np.zeros(E + 1, dtype=np.int64)
    off[1:] = np.cumsum(padded)
    num_padded = int(off[E])
    cap = align_capacity(A, E, B)
    sorted_ids = np.full(cap, A, dtype=np.int64)
    block_expert = np.full(cap // B if B else 0, -1, dtype=np.int64)
    for e in range(E):
        members = np.nonzero(flat == e)[0]          # ascending f
        sorted_ids[off[e]: off[e] + members.size] = members
        block_expert[off[e] // B: off[e + 1] // B] = e
    return {
        "counts": counts.astype(np.int32),
        "offsets": off.astype(np.int32),
        "sorted_ids": sorted_ids.astype(np.int32),
        "block_expert": block_expert.astype(np.int32),
        "num_padded": num_padded,
        "capacity": cap,
    }


# --------------------------------------------------------------------------
# Block-scaled FP8 activations (the W8A8 mode; [P2] §fp8)
# --------------------------------------------------------------------------

MX_BLOCK = 32          # values sharing one scale
E4M3_MAX = 448.0       # largest finite e4m3fn value
E4M3_EMAX = 8          # its exponent: 448 = 1.75 * 2^8
E8M0_EMIN, E8M0_EMAX = -127, 127   # exponents an 8-bit E8M0 scale holds (code 255 is NaN)

# the 127 non-negative finite e4m3fn values, ascending with their codes
# (code 0x7F is NaN); codes 0x00..0x7E are already in ascending value order
_E4M3_POS = np.array([_e4m3fn_value(c) for c in range(0x7F)], dtype=np.float64)


def _e4m3fn_nearest(y: np.ndarray) -> np.ndarray:
    """e4m3fn code nearest to each y with |y| <= 448; ties to the even code."""
    pos = _E4M3_POS
    a = np.abs(y)
    hi = np.clip(np.searchsorted(pos, a, side="left"), 0, pos.size - 1)
    lo = np.clip(hi - 1, 0, pos.size - 1)
    dlo = np.abs(a - pos[lo])
    dhi = np.abs(pos[hi] - a)
    pick = np.where(dlo < dhi, lo, np.where(dhi < dlo, hi, np.where(lo % 2 == 0, lo, hi)))
    codes = pick.astype(np.uint8)
    neg = np.signbit(y)                    # the sign is kept, also on zero
    return np.where(neg, codes | np.uint8(0x80), codes).astype(np.uint8)


def mx_quantize(v, block: int = MX_BLOCK):
    """Quantise each row of v [rows, K] (K a multiple of `block`) to e4m3fn
    codes with one power-of-two scale per block of consecutive values.

    For each block: amax = max |v|; the scale is X = 2^(floor(log2 amax) - 8)
    (8 is the exponent of e4m3fn's largest value), or X = 1 when amax = 0,
    with the exponent kept inside E8M0's range [-127, 127] (the scale is an
    8-bit exponent); each value becomes the e4m3fn code nearest to
    clamp(v / X, -448, 448), ties to the even code.  Returns (codes uint8
    [rows, K], exps int32 [rows, K / block]) with X = 2^exps.
    """
    v = np.asarray(v, dtype=np.float64)
    rows, K = v.shape
    if K % block:
        raise ValueError("K must be a multiple of the block")
    vb = v.reshape(rows, K // block, block)
    amax = np.abs(vb).max(axis=2)
    exps = np.zeros(amax.shape, dtype=np.int32)
    nz = amax > 0
    if nz.any():
        # floor(log2 amax) from the float's own exponent (exact at powers of two)
        _, e = np.frexp(amax[nz])          # amax = m * 2^e, m in [0.5, 1)
        exps[nz] = np.clip((e - 1).astype(np.int32) - E4M3_EMAX, E8M0_EMIN, E8M0_EMAX)
    y = vb / np.ldexp(1.0, exps)[:, :, None]
    y = np.clip(y, -E4M3_MAX, E4M3_MAX)
    codes = _e4m3fn_nearest(y.reshape(rows, K))
    return codes, exps


def mx_dequantize(codes, exps, block: int = MX_BLOCK) -> np.ndarray:
    """codes [rows, K], exps [rows, K / block] -> values, exactly."""
    vals = decode_e4m3fn(codes)
    rows, K = vals.shape
    sc = np.ldexp(1.0, np.asarray(exps, dtype=np.int64))
    return (vals.reshape(rows, K // block, block) * sc[:, :, None]).reshape(rows, K)


def _mx_roundtrip(v):
    return mx_dequantize(*mx_quantize(v))


# --------------------------------------------------------------------------
# Expert computation ([P2] §fused: "a szakértői hálózatok számításai")
# --------------------------------------------------------------------------

def silu(z: np.ndarray) -> np.ndarray:
    """SiLU(z) = z / (1 + e^-z) in fp64."""
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def expert_ffn(xrows: np.ndarray, w13: np.ndarray, w2: np.ndarray, h_quant=None,
               parts: dict | None = None) -> np.ndarray:
    """One expert's SwiGLU network on a batch of rows.

    xrows [n, d]; w13 [2I, d] with rows 0..I-1 the gate projection W1 and rows
    I..2I-1 the up projection W3; w2 [d, I].  Returns [n, d]:
    W2 . (SiLU(W1 x) * (W3 x)) for every row x.  `h_quant`, when given, maps
    the rows of SiLU(W1 x) * (W3 x) to the values W2 sees (the W8A8 mode's
    quantise-dequantise step).  `parts`, when given, receives the
    intermediates: "g" = W1 x, "u" = W3 x, "h" = SiLU(g) * u and "h_used"
    (what W2 multiplies: h, or its quantised values), each [n, I].
    """
    I = w13.shape[0] // 2
    g = xrows @ w13[:I].T
    u = xrows @ w13[I:].T
    h = silu(g) * u
    hq = h_quant(h) if h_quant is not None else h
    if parts is not None:
        parts.update(g=g, u=u, h=h, h_used=hq)
    return hq @ w2.T


# --------------------------------------------------------------------------
# The layer: the per-expert loop the fused operation replaces
# --------------------------------------------------------------------------

def moe_forward(x, w_gate, w13, w2, top_k: int, *, act_fmt: str = "bf16",
                w_fmt: str = "bf16", s13=None, s2=None, scale_mode: str | None = None,
                block_m: int = 64, logits=None, act_quant: str | None = None,
                expert_hook=None, workers: int = 1) -> dict:
    """The MoE layer computed as a plain loop over experts.

    x: [T, d] raw activations (uint16 bf16 patterns or float32);
    w_gate: [E, d] float32;
    w13[e]: [2I, d] raw weights of expert e; w2[e]: [d, I] raw weights
      (any object whose [e] gives the expert's array works, so callers may
      fetch experts lazily -- only experts that receive tokens are read);
    s13, s2: e4m3fn scales, [E, 2I] and [E, d] per channel or [E] per tensor;
    logits: optional [T, E] router logits to use instead of computing them
      (used to compare routing given identical logits);
    act_quant: None (activations as given) or "mx_e4m3" (the W8A8 mode: the
      router still sees x as given; the experts see x quantised per token
      and h quantised per routing slot by mx_quantize, then dequantised);
    expert_hook: optional callable, called once per expert that receives
      slots, after its network has run, with a dict of what the loop has at
      hand: "e", "slots" (flat slot ids f, ascending), "x" (the rows the
      expert saw [n, d]), "w13" [2I, d] and "w2" [d, I] (decoded fp64
      values), "gates" [n], and the intermediates of expert_ffn ("g", "u",
      "h", "h_used", [n, I]).  It observes only: nothing it returns is used.
    workers: experts are independent, so with workers > 1 their networks
      run in a pool of that many threads (each writes only its own slots'
      rows; the hook may then be called from several threads at once).  The
      arithmetic of each expert is the same either way.

    Steps: (1) logits, (2) top-k selection and gates, (3) regrouping by expert,
    (4) for each expert, gather its tokens, run its SwiGLU network and scale
    each row by its gate, (5) out[t] = sum over the k slots of t in rank order.
    Everything stays fp64; the returned ``out`` is not rounded to the
    activation format.
    """
    xv = _decode_act(x, act_fmt)
    if xv.ndim != 2:
        raise ValueError("x must be [T, d]")
    T, d = xv.shape
    wg = np.asarray(w_gate, dtype=np.float32)
    E = wg.shape[0]
    if logits is None:
        lg = router_logits(xv, wg)
    else:
        lg = np.asarray(logits, dtype=np.float64)
    k = int(top_k)
    if T:
        ids = select_topk(lg, k)
        gates = gate_weights(lg, ids)
    else:
        if not 1 <= k <= E:
            raise ValueError(f"top_k must be in [1, {E}], got {k}")
        ids = np.zeros((0, k), dtype=np.int32)
        gates = np.zeros((0, k), dtype=np.float64)
    al = align(ids, E, block_m)
    A = T * k
    y_slot = np.zeros((A, d), dtype=np.float64)
    flat_gates = gates.reshape(-1)

    if w_fmt == "e4m3fn":
        if scale_mode not in ("channel", "tensor"):
            raise ValueError("e4m3fn weights need scale_mode 'channel' or 'tensor'")
    if act_quant not in (None, "mx_e4m3"):
        raise ValueError(f"unknown act_quant {act_quant!r}")
    xe = _mx_roundtrip(xv) if (act_quant and T) else xv   # what the experts see
    hq = _mx_roundtrip if act_quant else None

    def run_expert(e: int) -> None:
        n = int(al["counts"][e])
        start = int(al["offsets"][e])
        fs = al["sorted_ids"][start:start + n].astype(np.int64)
        ts = fs // k
        if w_fmt == "e4m3fn":
            sc13 = np.asarray(s13[e])
            sc2 = np.asarray(s2[e])
        else:
            sc13 = sc2 = None
        W13e = decode_weights(w13[e], w_fmt, sc13)
        W2e = decode_weights(w2[e], w_fmt, sc2)
        if W13e.shape[1] != d or W2e.shape[0] != d or W13e.shape[0] != 2 * W2e.shape[1]:
            raise ValueError("weight shapes do not match x / each other")
        parts = {} if expert_hook is not None else None
        Y = expert_ffn(xe[ts], W13e, W2e, hq, parts)
        y_slot[fs] = flat_gates[fs][:, None] * Y
        if expert_hook is not None:
            expert_hook(dict(e=e, slots=fs, x=xe[ts], w13=W13e, w2=W2e,
                             gates=flat_gates[fs], **parts))

    live = [e for e in range(E) if int(al["counts"][e]) > 0]
    if workers > 1 and len(live) > 1:
        import concurrent.futures
        with concurrent.futures.ThreadPoolExecutor(max_workers=int(workers)) as pool:
            for _ in pool.map(run_expert, live):
                pass
    else:
        for e in live:
            run_expert(e)

    out = np.zeros((T, d), dtype=np.float64)
    ys = y_slot.reshape(T, k, d)
    for j in range(k):
        out += ys[:, j, :]
    return {
        "out": out,
        "logits": lg,
        "ids": ids,
        "gates": gates,
        "y_slot": y_slot,
        **al,
    }
