"""Plain CPU oracle of the sparse MoE block forward (test infrastructure only).

Only the test-suite, the package smoke check and the benchmark's CPU-baseline
leg may import this module. It shares no code with the HIP path: it has its
own codecs (``oracle.codecs``) and consumes the same generated input bytes.

The block, as the "GPT-OSS on day 0" post defines it (section "GPT-OSS on
Hopper": sparse MoE MLP, SwiGLU activation, softmax after top-k for the
expert weights, experts with biases; FP8 with 128x128 block scaling) and its
section "MoE" (routing picks the top-k experts and the softmax runs over the
selected ones only; tokens are dispatched to their experts and combined by a
weighted accumulation):

1. decode bf16 / e4m3 inputs exactly to fp64;
2. router logits ``l = x @ W_router + b_router`` (fp64);
3. top-k: the k largest logits per token, descending, ties to the lower
   expert index;
4. gate weights: stabilised softmax (the max-subtracted form given in the
   section "Sink attention") over the k selected logits, fp64;
5. counting-sort permutation of the (token, slot) pairs by expert, stable in
   token order;
6. activation quantisation of x per token per 128-column group, in fp32:
   ``s = fl32(amax/448)`` (1.0 for an all-zero group), ``q = e4m3(fl32(x/s))``;
7. per expert: ``P = deq(xq) @ deq(W_gateup) + b_gateup`` (fp64), columns
   [0,f) gate and [f,2f) up; ``h = silu(gate) * up``;
8. ``fl32(h)`` quantised per row per 128 columns like step 6;
9. ``Y = deq(hq) @ deq(W_down) + b_down`` (fp64);
10. ``out[t] = sum_j w[t,j] * Y[row(t,j)]`` in fp64, not rounded.

MXFP8 variant (``inp["format"] == "mx"``; the "Hosting Qwen on Blackwell"
post, section "Quantization", names microscaling as the Blackwell format,
with the weights converted statically): steps 6 and 8 quantise per row per
32 columns with a power-of-two E8M0 scale, and the weights carry one E8M0
scale per 32 rows of K per column; everything else is unchanged.  MXFP4 weights
(``"mxfp4"``; the post's section "GPT-OSS on Hopper" says the checkpoints ship
in MXFP4): the weights are E2M1 with the same E8M0 scale blocks, two codes per
byte along K; the activations are MXFP8 as above.

Readings of points the pages leave open are listed in the repository's
design notes; each is marked "reading:" below where it is taken.

Parity pins: every step is pinned by a CPU test against something other than
itself (format definition points, brute force, closed forms, a library
special case, a dense-MLP reduction, all-experts brute force, invariants).
The complete output has no printed worked example on the pages: beyond those
pins it is "parity unpinned".
"""
from __future__ import annotations

import numpy as np

from .codecs import (E8M0_BIAS, bf16_decode, e2m1_decode, e4m3_decode, e4m3_encode_rne, e8m0_decode,
                     unpack_fp4_k)

GROUP = 128
MX_GROUP = 32
FP8_MAX = np.float32(448.0)


# ----------------------------------------------------------------------------- routing
def router_logits(x_bits: np.ndarray, W_router: np.ndarray, b_router: np.ndarray) -> np.ndarray:
    """Router scores with bias, fp64: ``x @ W_router + b_router`` [T, E]."""
    return bf16_decode(x_bits) @ np.asarray(W_router, np.float64) + np.asarray(b_router, np.float64)


def topk_select(logits: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest logits per row, descending (ties: lower index first).

    Reading: the pages fix neither order nor ties; only the selected set
    matters for the output.
    """
    T, E = logits.shape
    order = np.lexsort((np.broadcast_to(np.arange(E), (T, E)), -logits), axis=1)
    return order[:, :k].astype(np.int32)


def gate_weights(logits: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """Softmax over the k selected logits only ("GPT-OSS on day 0", section "MoE"),
    in the max-subtracted form of section "Sink attention". fp64 [T, k]."""
    sel = np.take_along_axis(logits, idx, axis=1)
    z = np.exp(sel - sel.max(axis=1, keepdims=True))
    return z / z.sum(axis=1, keepdims=True)


def gate_weights_all(logits: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """Routing variant: the softmax is taken over all E logits before top-k
    (the DeepSeek-style rule that "GPT-OSS on day 0", section "MoE", contrasts
    with gpt-oss's softmax over the selected experts).  Reading: the selected
    experts keep their full-softmax probabilities, not renormalised over the
    k.  Max-subtracted form, fp64 [T, k]."""
    z = np.exp(logits - logits.max(axis=1, keepdims=True))
    p = z / z.sum(axis=1, keepdims=True)
    return np.take_along_axis(p, idx, axis=1)


def bf16_round_weights(w: np.ndarray) -> np.ndarray:
    """Gate weights rounded to bf16 (round to nearest even), as fp64.  The
    section "MoE" calls for the expert weights in bf16 (reading: an option;
    the default keeps them in fp32 on the GPU and fp64 here)."""
    from .codecs import bf16_round
    return bf16_round(np.asarray(w, np.float64))


def permutation(idx: np.ndarray, E: int):
    """Expert-contiguous order of the routed (token, slot) pairs.

    Counting sort by expert, stable in token order (reading: rows of one
    expert ascend in token index; offsets are not padded).  Returns
    counts [E], offsets [E+1] (exclusive scan), row_of [T,k] (row of each
    pair) and row_token [T*k] (token of each row).
    """
    T, k = idx.shape
    flat = idx.reshape(-1).astype(np.int64)
    counts = np.bincount(flat, minlength=E).astype(np.int32)
    offsets = np.zeros(E + 1, np.int32)
    offsets[1:] = np.cumsum(counts)
    order = np.argsort(flat, kind="stable")           # pairs in (expert, token) order
    row_of = np.empty(T * k, np.int32)
    row_of[order] = np.arange(T * k, dtype=np.int32)
    row_token = (order // k).astype(np.int32)
    return counts, offsets, row_of.reshape(T, k), row_token


# ----------------------------------------------------------------------------- quantisation
def quantize_groups(v: np.ndarray):
    """Per-row 1x128 e4m3 quantisation of fp32 values ``v`` [N, K].

    Reading: scale ``s = fl32(amax/448)`` (not a power of two), ``s = 1`` for
    an all-zero group, codes ``e4m3_rne(clamp(fl32(v/s), +-448))``; the
    arithmetic is IEEE fp32 (NumPy float32 division is correctly rounded).
    Returns (codes uint8 [N, K], scales fp32 [N, K/128]).
    """
    v = np.asarray(v, dtype=np.float32)
    N, K = v.shape
    g = v.reshape(N, K // GROUP, GROUP)
    amax = np.abs(g).max(axis=2) if N * K else np.zeros((N, K // GROUP), np.float32)
    s = np.where(amax > 0, amax / FP8_MAX, np.float32(1.0)).astype(np.float32)
    y = (g / s[:, :, None]).astype(np.float32)
    y = np.clip(y, -FP8_MAX, FP8_MAX)
    return e4m3_encode_rne(y).reshape(N, K), s


def dequant_groups(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Inverse of ``quantize_groups`` in fp64: code value times its group scale."""
    N, K = codes.shape
    return (e4m3_decode(codes).reshape(N, K // GROUP, GROUP)
            * np.asarray(scales, np.float64)[:, :, None]).reshape(N, K)


def dequant_weight(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """One expert's e4m3 matrix [K, N] times its 128x128 block scales -> fp64."""
    K, N = codes.shape
    blk = np.asarray(scales, np.float64)
    return (e4m3_decode(codes).reshape(K // GROUP, GROUP, N // GROUP, GROUP)
            * blk[:, None, :, None]).reshape(K, N)


# ----------------------------------------------------------------------------- MXFP8
#: 448 * 2^e for every exponent an E8M0 code can hold (1..254 -> -126..127, and 0 -> -127)
_MX_EXPONENTS = np.arange(-E8M0_BIAS, E8M0_BIAS + 1)
_MX_LIMITS = 448.0 * np.ldexp(1.0, _MX_EXPONENTS)


def mx_scale_exponent(amax: np.ndarray) -> np.ndarray:
    """Exponent e of the E8M0 scale 2^e of an MX block with largest magnitude ``amax``.

    Reading: e is the smallest exponent with ``amax <= 448 * 2^e``, so no
    element of the block saturates (the common Blackwell MXFP8 recipe); the
    OCP rule floor(log2 amax) - 8 may clip the largest elements instead.  An
    all-zero block gets the smallest scale, 2^-127.  Exact: the comparison
    runs on fp64 values that hold 448 * 2^e and every fp32 amax exactly.
    """
    a = np.asarray(amax, dtype=np.float64)
    i = np.searchsorted(_MX_LIMITS, a.reshape(-1), side="left")
    return _MX_EXPONENTS[np.minimum(i, len(_MX_LIMITS) - 1)].reshape(a.shape)


def quantize_mx(v: np.ndarray):
    """Per-row 1x32 MXFP8 quantisation of fp32 values ``v`` [N, K].

    ``X = 2^e`` (``mx_scale_exponent`` of the block's amax), codes
    ``e4m3_rne(v / X)``: the division by a power of two is exact, and
    ``|v / X| <= 448`` by the choice of e.  Returns (codes uint8 [N, K],
    E8M0 scale codes uint8 [N, K/32] = e + 127).
    """
    v = np.asarray(v, dtype=np.float32)
    N, K = v.shape
    g = v.reshape(N, K // MX_GROUP, MX_GROUP).astype(np.float64)
    amax = np.abs(g).max(axis=2) if N * K else np.zeros((N, K // MX_GROUP))
    e = mx_scale_exponent(amax)
    codes = e4m3_encode_rne(g / np.ldexp(1.0, e)[:, :, None])
    return codes.reshape(N, K), (e + E8M0_BIAS).astype(np.uint8)


def dequant_mx(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Inverse of ``quantize_mx`` in fp64: code value times its block's 2^e."""
    N, K = codes.shape
    return (e4m3_decode(codes).reshape(N, K // MX_GROUP, MX_GROUP)
            * e8m0_decode(scales)[:, :, None]).reshape(N, K)


def dequant_weight_mx(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """One expert's e4m3 matrix [K, N] times its E8M0 scales [K/32, N] (one per
    32 rows of K per column: the MX blocks run along the contraction) -> fp64."""
    K, N = codes.shape
    return (e4m3_decode(codes).reshape(K // MX_GROUP, MX_GROUP, N)
            * e8m0_decode(scales)[:, None, :]).reshape(K, N)


def dequant_weight_mxfp4(packed: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """One expert's MXFP4 matrix: e2m1 codes packed two per byte along K
    ([K/2, N], low nibble = even K) times E8M0 scales [K/32, N] -> fp64 [K, N]."""
    codes = unpack_fp4_k(packed)
    K, N = codes.shape
    return (e2m1_decode(codes).reshape(K // MX_GROUP, MX_GROUP, N)
            * e8m0_decode(scales)[:, None, :]).reshape(K, N)


#: quantise activations, dequantise them, dequantise one expert's weights
FORMATS = {
    "block128": (quantize_groups, dequant_groups, dequant_weight),
    "mx": (quantize_mx, dequant_mx, dequant_weight_mx),
    "mxfp4": (quantize_mx, dequant_mx, dequant_weight_mxfp4),
}


# ----------------------------------------------------------------------------- experts
def silu(z: np.ndarray) -> np.ndarray:
    """z * sigmoid(z), fp64."""
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def expert_mlp(xdeq: np.ndarray, Wgu_e, Sgu_e, bgu_e, Wdn_e, Sdn_e, bdn_e, return_h=False,
               fmt="block128"):
    """One expert on its rows: biased gate/up projection, SwiGLU, h quantisation,
    biased down projection ("GPT-OSS on day 0", section "GPT-OSS on Hopper":
    SwiGLU experts with biases; section "MoE": the bias sits in the GEMM).
    ``fmt`` picks the FP8 scaling (``FORMATS``).

    Reading: columns [0,f) of the gate/up matrix are the gate, [f,2f) the up
    projection; h is rounded to fp32 before its quantisation.
    """
    quant, deq, wdeq = FORMATS[fmt]
    f = Wgu_e.shape[1] // 2
    P = xdeq @ wdeq(Wgu_e, Sgu_e) + bf16_decode(bgu_e)
    h = silu(P[:, :f]) * P[:, f:]
    hq, hs = quant(h.astype(np.float32))
    Y = deq(hq, hs) @ wdeq(Wdn_e, Sdn_e) + bf16_decode(bdn_e)
    if return_h:
        return Y, P, h, hq, hs
    return Y


def route(inp: dict):
    """Steps 2-5 for all tokens.  Optional keys of ``inp``: ``routing`` =
    "topk_softmax" (default: softmax over the selected logits) or
    "softmax_topk" (softmax over all logits, ``gate_weights_all``), and
    ``gate_bf16`` (round the gate weights to bf16)."""
    logits = router_logits(inp["x"], inp["W_router"], inp["b_router"])
    idx = topk_select(logits, inp["k"])
    routing = inp.get("routing", "topk_softmax")
    if routing == "topk_softmax":
        w = gate_weights(logits, idx)
    elif routing == "softmax_topk":
        w = gate_weights_all(logits, idx)
    else:
        raise ValueError(f"unknown routing {routing!r}")
    if inp.get("gate_bf16", False):
        w = bf16_round_weights(w)
    counts, offsets, row_of, row_token = permutation(idx, inp["E"])
    return dict(logits=logits, idx=idx, w=w, counts=counts, offsets=offsets,
                row_of=row_of, row_token=row_token)


def forward(inp: dict, tokens=None, keep=False):
    """The whole block. ``tokens`` (optional) restricts the expert work and the
    output to a subset of tokens; routing and permutation cover all tokens.

    ``inp["format"]`` (optional): "block128" (default), "mx" or "mxfp4".

    Returns a dict: out64 [len(tokens), d] fp64 (unrounded), routing arrays,
    xq/xs for the evaluated tokens, and (with ``keep``) per-row intermediates.
    """
    T, k, E = inp["T"], inp["k"], inp["E"]
    fmt = inp.get("format", "block128")
    quant, deq, _ = FORMATS[fmt]
    r = route(inp)
    tok = np.arange(T) if tokens is None else np.asarray(tokens, dtype=np.int64)
    x32 = bf16_decode(inp["x"][tok]).astype(np.float32)
    xq, xs = quant(x32)
    xdeq = deq(xq, xs)
    d = inp["d"]
    out = np.zeros((len(tok), d))
    inter = {}
    sel_idx = r["idx"][tok]
    for e in range(E):
        pos, slot = np.nonzero(sel_idx == e)              # evaluated tokens routed to e
        if len(pos) == 0:
            continue
        res = expert_mlp(xdeq[pos], inp["W_gateup"][e], inp["S_gateup"][e], inp["b_gateup"][e],
                         inp["W_down"][e], inp["S_down"][e], inp["b_down"][e], return_h=keep,
                         fmt=fmt)
        Y = res[0] if keep else res
        np.add.at(out, pos, r["w"][tok[pos], slot][:, None] * Y)
        if keep:
            rows = r["row_of"][tok[pos], slot]
            inter[e] = dict(rows=rows, Y=Y, P=res[1], h=res[2], hq=res[3], hs=res[4])
    res = dict(out64=out, tokens=tok, xq=xq, xs=xs, **r)
    if keep:
        res["experts"] = inter
    return res
