"""Routing, permutation and the fused MoE layer (oracle; test infrastructure).

The layer, as the pages describe the fused kernels: one call performs the
routing, token dispatch, W1 (gate/up) GEMM, SwiGLU, W2 (down) GEMM and the
reduction over the selected experts; bf16 hidden states go in and are
quantised inside [vLLM PR 40082 report, "Implementation" item 1 and "Key
source excerpts"; MegaMoE drop workflow, §1, the three numeric formats].

Readings where the pages are silent (all documented with the design):

1. Router logits are an input; scoring is softmax over the selected top-k
   (renormalised), which equals softmax over all experts restricted to the
   top-k and renormalised.
2. Selection order: logit descending, ties to the lower expert id; slot j of
   a token is its j-th pick.  -0 and +0 tie.  Non-finite logits are rejected.
3. W13 rows [0, I) are the gate projection, rows [I, 2I) the up projection
   (the pages note that producers disagree on the gate/up order: [vLLM PR
   40082 report, "Implementation" item 5, the reorder helper in the test]).
4. SwiGLU: h = silu(g) * u = g / (1 + exp(-g)) * u; no clamp, no bias.
5. The intermediate h is requantised in the layer's format before the down
   GEMM (bf16: round to nearest even; MXFP8 / NVFP4: the dynamic block rules
   with global scale 1), the decision taken on fp32 h (kernel precision).
6. Combine: out_t = bf16( sum_j w_tj * y_tj ), summed in slot order; no shared
   expert, no linear biases, no token dropping.
7. Layer format "bf16_mxfp8" (the pages list a bf16 x MXFP8 MegaMoE entry
   beside the three formats [MegaMoE drop workflow, §1, the package exports]
   and say nothing more): MXFP8 weights with the activation path of the BF16
   layer -- x is used as given and the intermediate is rounded to bf16.
8. ReLU^2 experts (the pages note that models with squared-ReLU, non-gated
   experts, such as Nemotron, are rejected by the b12x backend [vLLM PR 40082
   report, "Risks" item 4]): W1 = W13 holds I rows and h = relu(W1 x)^2,
   requantised like the SwiGLU intermediate; the rest of the layer is the same.
9. Gate/up clamp (the pages name a resolve_gate_up_clamp step of the kernels'
   adaptation layer and give no value or rule [MegaMoE drop workflow, §2, the
   shim/comm.py entry]): an optional limit L > 0 of the SwiGLU experts, applied
   to the fp32 products before the activation, gate = min(gate, L) and
   up = clamp(up, -L, L) (the gate bounded from above only, since silu of a
   very negative gate already vanishes); L = 0 means no clamp.

Arithmetic: dequantised operands are exact in float64, dot products and the
SwiGLU are evaluated in float64, and rounding to fp32 happens only where the
layer stores a quantised value (requantisation of h, the bf16 output).
"""
from __future__ import annotations

import dataclasses

import numpy as np

from . import codecs, quant

# ------------------------------------------------------------------ routing


def route(logits: np.ndarray, k: int):
    """Top-k softmax routing [vLLM PR 40082 report, "Implementation" item 1].

    logits fp32 [T, E] -> (ids int32 [T, k], weights float64 [T, k]).
    ids[t, j] is the j-th expert in (logit descending, id ascending) order;
    weights are exp(l - l_max) normalised over the k picks.
    """
    l = np.asarray(logits, np.float32).astype(np.float64)
    if l.ndim != 2 or not (1 <= k <= l.shape[1]):
        raise ValueError("bad routing shape")
    if not np.all(np.isfinite(l)):
        raise ValueError("non-finite router logit")
    # +0.0 turns -0.0 into +0.0 so the two tie; a stable sort keeps lower ids first
    order = np.argsort(-l + 0.0, axis=1, kind="stable")
    ids = order[:, :k].astype(np.int32)
    sel = np.take_along_axis(l, ids.astype(np.int64), axis=1)
    ex = np.exp(sel - sel[:, :1])
    return ids, ex / ex.sum(axis=1, keepdims=True)


# ------------------------------------------------------------------ permutation


def permute(ids: np.ndarray, E: int):
    """Token dispatch as a permutation of (token, slot) pairs by expert
    [vLLM PR 40082 report, "Key source excerpts", class docstring: token
    dispatch fused with the GEMMs].

    Pair p = t * k + j.  Returns (offsets int32 [E+1], sorted_pairs int32 [P],
    pair_pos int32 [P]): offsets is the exclusive prefix sum of per-expert
    counts, sorted_pairs the pairs in (expert, p) order, pair_pos its inverse.
    """
    flat = np.asarray(ids, np.int64).ravel()
    if flat.size and (flat.min() < 0 or flat.max() >= E):
        raise ValueError("expert id out of range")
    counts = np.bincount(flat, minlength=E)
    offsets = np.zeros(E + 1, np.int64)
    np.cumsum(counts, out=offsets[1:])
    sorted_pairs = np.argsort(flat, kind="stable")
    pair_pos = np.empty_like(sorted_pairs)
    pair_pos[sorted_pairs] = np.arange(flat.size)
    return offsets.astype(np.int32), sorted_pairs.astype(np.int32), pair_pos.astype(np.int32)


# ------------------------------------------------------------------ formats


def weight_format(fmt: str) -> str:
    """The format of a layer format's weights."""
    return "mxfp8" if fmt == "bf16_mxfp8" else fmt


def act_format(fmt: str) -> str:
    """The format of a layer format's activations (x and the intermediate)."""
    return "bf16" if fmt == "bf16_mxfp8" else fmt


# ------------------------------------------------------------------ weights


@dataclasses.dataclass
class Weights:
    """Canonical quantised expert weights.

    dtype bf16:  w13 uint16 [E, 2I, H], w2 uint16 [E, H, I]
    dtype mxfp8: w13 e4m3 [E, 2I, H] + w13_s e8m0 [E, 2I, H/32]; same for w2
    dtype nvfp4: w13 packed e2m1 [E, 2I, H/2] + w13_s e4m3 [E, 2I, H/16]
                 + w13_a fp32 [E]; same for w2
    dtype bf16_mxfp8: as mxfp8 (the layer format's weights)
    Any of the per-expert arrays may be a mapping {expert: array} holding only
    the experts a computation needs.  act "swiglu": W13 rows [0, I) gate,
    [I, 2I) up; act "relu2": W13 is W1 of I rows.
    """

    dtype: str
    w13: object
    w2: object
    w13_s: object = None
    w2_s: object = None
    w13_a: object = None
    w2_a: object = None
    act: str = "swiglu"
    limit: float = 0.0  # gate/up clamp of SwiGLU experts (0: none)

    def dequant(self, e: int):
        """Exact float64 dequantised (W13 [2I, H], W2 [H, I]) of expert e."""
        def g(x):
            return None if x is None else x[e]

        wf = weight_format(self.dtype)
        w13 = quant.dequantize_weight(g(self.w13), g(self.w13_s), g(self.w13_a), wf)
        w2 = quant.dequantize_weight(g(self.w2), g(self.w2_s), g(self.w2_a), wf)
        return w13, w2


def quantize_weights(w13_f32: dict, w2_f32: dict, dtype: str, act: str = "swiglu", fold: bool = False,
                     limit: float = 0.0) -> Weights:
    """Quantise fp32 master weights {e: array} into canonical form (harness).
    fold (NVFP4): then fold each tensor's alpha into its block scales.
    limit: the experts' gate/up clamp (0: none)."""
    out = {k: {} for k in ("w13", "w13_s", "w13_a", "w2", "w2_s", "w2_a")}
    wf = weight_format(dtype)
    for e in w13_f32:
        out["w13"][e], out["w13_s"][e], out["w13_a"][e] = quant.quantize_weight(w13_f32[e], wf)
        out["w2"][e], out["w2_s"][e], out["w2_a"][e] = quant.quantize_weight(w2_f32[e], wf)
    if fold and wf == "nvfp4":
        for e in w13_f32:
            out["w13_s"][e], out["w13_a"][e] = quant.nvfp4_fold_global_scale(out["w13_s"][e], out["w13_a"][e])
            out["w2_s"][e], out["w2_a"][e] = quant.nvfp4_fold_global_scale(out["w2_s"][e], out["w2_a"][e])
    if wf == "bf16":
        for n in ("w13_s", "w13_a", "w2_s", "w2_a"):
            out[n] = None
    if wf == "mxfp8":
        out["w13_a"] = out["w2_a"] = None
    return Weights(dtype=dtype, act=act, limit=float(limit), **out)


# ------------------------------------------------------------------ the layer


def silu_mul(g: np.ndarray, u: np.ndarray, limit: float = 0.0) -> np.ndarray:
    """SwiGLU activation silu(g) * u (act_and_mul) [vLLM PR 40082 report,
    "Implementation" item 1; "Risks" item 4: only gated act-and-mul MLPs],
    after the optional gate/up clamp (reading 9): with limit L > 0 the gate is
    min(g, L) and the up value is clamped to [-L, L]."""
    if limit > 0:
        g = np.minimum(g, limit)
        u = np.clip(u, -limit, limit)
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g)) * u


def relu2(g: np.ndarray) -> np.ndarray:
    """Squared ReLU activation of non-gated experts: max(g, 0)^2."""
    r = np.maximum(g, 0.0)
    return r * r


def requant_h(h64: np.ndarray, dtype: str):
    """Requantise the intermediate in the layer format's activation format
    (decision on fp32 h); returns (codes, scales, dequantised float64)."""
    dtype = act_format(dtype)
    h32 = np.asarray(h64, np.float64).astype(np.float32)
    c, s = quant.quantize_act(h32, dtype)
    return c, s, quant.dequantize_act(c, s, dtype)


def quantize_x(x_bits: np.ndarray, dtype: str):
    """In-kernel activation quantisation of bf16 hidden states in the layer
    format's activation format; returns (codes, scales, dequantised float64).
    bf16 passes through."""
    dtype = act_format(dtype)
    x32 = codecs.bf16_decode(x_bits).astype(np.float32)
    c, s = quant.quantize_act(x32, dtype)
    if dtype == "bf16":
        c = np.asarray(x_bits, np.uint16)
    return c, s, quant.dequantize_act(c, s, dtype)


def expert_mlp(xh: np.ndarray, w13: np.ndarray, w2: np.ndarray, act: str, dtype: str, limit: float = 0.0):
    """One routed pair through its expert: xh the dequantised activation row
    (float64 [H]), w13 / w2 the expert's dequantised weights.  Gate/up product,
    SwiGLU (or squared ReLU), requantisation of the intermediate in the layer
    format, down product.  Returns ((codes, scales, dequantised) of the
    intermediate, y float64 [H])."""
    if act == "relu2":
        h = relu2(w13 @ xh)
    else:
        I = w13.shape[0] // 2
        h = silu_mul(w13[:I] @ xh, w13[I:] @ xh, limit)
    hc, hsc, hh = requant_h(h[None, :], dtype)
    y = w2 @ hh[0]
    return (hc[0], None if hsc is None else hsc[0], hh[0]), y


def batched_experts(x_bits: np.ndarray, counts, W: Weights):
    """The expert MLPs on tokens that arrive already bucketed per expert (the
    batched activation format of the CuteDSL batched-experts class [vLLM PR
    38050 report, "Implementation": FlashInferCuteDSLBatchedExperts, batched
    activation format, workspace_shapes]): no routing and no combine.

    x_bits bf16 [E, M, H]; counts [E] (values clamped to [0, M]).  Row r of
    expert e (r < counts[e]) is quantised, run through expert e's MLP (gate/up
    product, activation, requantisation, down product) and returned as
    y float64 [E, M, H]; the other rows of y are zero.
    """
    x_bits = np.asarray(x_bits, np.uint16)
    E, M, H = x_bits.shape
    y = np.zeros((E, M, H), np.float64)
    for e in range(E):
        c = int(min(max(int(counts[e]), 0), M))
        if c == 0:
            continue
        w13, w2 = W.dequant(e)
        _, _, xh = quantize_x(x_bits[e, :c], W.dtype)
        for r in range(c):
            _, y[e, r] = expert_mlp(xh[r], w13, w2, W.act, W.dtype, W.limit)
    return y


@dataclasses.dataclass
class LayerResult:
    out: np.ndarray            # bf16 bits [T, H] (rows of the requested tokens)
    out_f64: np.ndarray        # the fp64 sum before the bf16 rounding
    ids: np.ndarray
    weights: np.ndarray
    y: dict                    # (t, j) -> float64 [H] expert output
    h: dict                    # (t, j) -> (codes, scales, dequant) of the intermediate


def moe_layer(x_bits, logits, W: Weights, k: int, tokens=None, keep=False) -> LayerResult:
    """The layer as a literal per-token loop (the definition).

    x_bits bf16 [T, H], logits fp32 [T, E].  `tokens` restricts the work to a
    subset of tokens (every token is independent); the result rows follow
    `tokens` order.
    """
    x_bits = np.asarray(x_bits, np.uint16)
    T, H = x_bits.shape
    ids, wts = route(logits, k)
    toks = range(T) if tokens is None else list(tokens)
    out64 = np.zeros((len(toks), H), np.float64)
    ys, hs = {}, {}
    cache = {}
    for row, t in enumerate(toks):
        _, _, xh = quantize_x(x_bits[t:t + 1], W.dtype)
        xh = xh[0]
        acc = np.zeros(H, np.float64)
        for j in range(k):
            e = int(ids[t, j])
            if e not in cache:
                cache[e] = W.dequant(e)
            w13, w2 = cache[e]
            hq, y = expert_mlp(xh, w13, w2, W.act, W.dtype, W.limit)
            acc += wts[t, j] * y
            if keep:
                ys[(t, j)] = y
                hs[(t, j)] = hq
        out64[row] = acc
    out = codecs.bf16_encode(out64.astype(np.float32))
    return LayerResult(out, out64, ids, wts, ys, hs)


def moe_layer_grouped(x_bits, logits, W: Weights, k: int, acc_dtype=np.float64):
    """The same layer, expert-grouped: per expert, one matrix product over all
    pairs routed to it (BLAS), then the slot-order weighted sum.

    acc_dtype float32 gives an fp32-accumulating variant (used to show how far
    accumulation precision moves the result).
    """
    x_bits = np.asarray(x_bits, np.uint16)
    T, H = x_bits.shape
    ids, wts = route(logits, k)
    E = int(np.asarray(logits).shape[1])
    offsets, sorted_pairs, _ = permute(ids, E)
    _, _, xh = quantize_x(x_bits, W.dtype)
    xh = xh.astype(acc_dtype)
    y = np.zeros((T * k, H), np.float64)
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if lo == hi:
            continue
        pairs = sorted_pairs[lo:hi]
        w13, w2 = W.dequant(e)
        X = xh[pairs // k]
        if W.act == "relu2":
            Hm = relu2((X @ w13.T.astype(acc_dtype)).astype(np.float64))
        else:
            I = w13.shape[0] // 2
            G = X @ w13[:I].T.astype(acc_dtype)
            U = X @ w13[I:].T.astype(acc_dtype)
            Hm = silu_mul(G.astype(np.float64), U.astype(np.float64), W.limit)
        _, _, hh = requant_h(Hm, W.dtype)
        y[pairs] = hh.astype(acc_dtype) @ w2.T.astype(acc_dtype)
    y = y.reshape(T, k, H)
    out64 = np.zeros((T, H), np.float64)
    for j in range(k):
        out64 += wts[:, j:j + 1] * y[:, j]
    out = codecs.bf16_encode(out64.astype(np.float32))
    return LayerResult(out, out64, ids, wts, {}, {})
