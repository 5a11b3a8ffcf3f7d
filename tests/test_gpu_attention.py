"""Sink attention: HIP kernels vs the CPU oracle through the C ABI (GPU only).

Gate (derived from the arithmetic): scores and the softmax run in fp32 and
the probabilities are rounded to bf16 (relative 2^-9) before the P.V
product, and the output is rounded to bf16, so every output element obeys
    |g - o| <= 2^-8 * (sum_j w_j |v_j|) + 2^-8 * |o| + 1e-6,
with w the oracle's softmax weights (sink included); sum_j w_j |v_j| is the
same attention applied to |v|.  The mean relative error sum|g - o| / sum|o|
is gated at 2^-8, the two bf16 roundings' combined worst case (2^-9 each);
typical values are near 2^-9 (the output rounding alone averages ~1.4e-3).
"""
import sys

import numpy as np
import pytest
import torch

import sparse_moe_layer_fp32_amd as moe
from oracle import attention as att
from sparse_moe_layer_fp32_amd import inputs as gen
from tests import parity

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _gate(g, o, absw, what):
    err = np.abs(g - o)
    bound = 2.0 ** -8 * absw + 2.0 ** -8 * np.abs(o) + 1e-6
    assert np.all(err <= bound), f"{what}: worst err/bound {(err / bound).max():.3f}"
    mean = err.sum() / max(np.abs(o).sum(), 1e-30)
    assert mean <= 2.0 ** -8, f"{what}: mean relative error {mean:.2e}"
    return float((err / bound).max()), float(mean)


def _abs_bits(b):
    return (np.asarray(b, np.uint16) & np.uint16(0x7FFF)).astype(np.uint16)


PREFILL = [
    # (S, Hq, Hkv): G = 8, 4, 2, 1, 16; ragged S; one token
    (1, 8, 1), (37, 8, 2), (64, 2, 1), (200, 4, 4), (130, 16, 2), (513, 64, 8), (300, 16, 1),
]


@pytest.mark.parametrize("S,Hq,Hkv", PREFILL, ids=[f"S{s}-Hq{a}-Hkv{b}" for s, a, b in PREFILL])
def test_prefill_vs_oracle(S, Hq, Hkv):
    inp = gen.make_attn_prefill(gen.AttnShape("t", Hq, Hkv), S, seed=S + Hq)
    _say(f"[attn prefill] S={S} Hq={Hq} Hkv={Hkv}")
    p = moe.attn_device_inputs(inp)
    out = moe.attn_prefill(p["q"], p["k"], p["v"], p["sinks"], p["sm_scale"])
    torch.cuda.synchronize()
    g = parity.bf16_to_f64(out)
    o = att.prefill(inp["q"], inp["k"], inp["v"], inp["sinks"], inp["sm_scale"])
    absw = att.prefill(inp["q"], inp["k"], _abs_bits(inp["v"]), inp["sinks"], inp["sm_scale"])
    _say("   err/bound, mean", _gate(g, o, absw, "prefill"))


DECODE = [
    # (B, Hq, Hkv, Lmax, lengths or None for seeded ragged lengths)
    (4, 8, 1, 300, None), (16, 64, 8, 1024, None), (3, 16, 1, 513, None), (5, 4, 4, 64, None),
    # the keys of all sequences are cut into equal ranges, one per wave (at least
    # 256 keys): ranges that start or end inside sequences and hold several
    # sequences, lengths 1 and 0 around them
    (6, 8, 2, 1100, [1, 256, 257, 1100, 1023, 513]),
    (24, 8, 8, 1500, [1, 512, 513, 1500, 1023, 1024] * 4),
    (40, 16, 8, 2000, None),
    (48, 8, 8, 2100, [1, 2048, 2049, 2100, 1024, 1025] * 8),
    (300, 8, 8, 600, None),                          # ranges of about 1000 keys over 2-4 sequences
    (9, 8, 8, 700, [0, 5, 0, 700, 1, 0, 300, 0, 2]),
    # long caches: a sequence in up to a few hundred ranges, merged by four waves
    (2, 8, 1, 40000, [40000, 9000]),
    (3, 16, 2, 20000, [20000, 1, 9999]),
    (1, 64, 8, 65536, [65536]),
    (70, 8, 1, 9000, None),                          # two chunks of sequences, four-wave merge
]


@pytest.mark.parametrize("B,Hq,Hkv,Lmax,lens", DECODE, ids=[f"B{d[0]}-Hq{d[1]}-Hkv{d[2]}-L{d[3]}" for d in DECODE])
def test_decode_vs_oracle(B, Hq, Hkv, Lmax, lens):
    inp = gen.make_attn_decode(gen.AttnShape("t", Hq, Hkv), B, Lmax, seed=B + Lmax)
    if lens is not None:
        inp["kv_len"] = np.asarray(lens, np.int32)
    _say(f"[attn decode] B={B} Hq={Hq} Hkv={Hkv} Lmax={Lmax} kv_len={inp['kv_len'].tolist()}")
    p = moe.attn_device_inputs(inp)
    out = moe.attn_decode(p["q"], p["k"], p["v"], p["kv_len"], p["sinks"], p["sm_scale"])
    torch.cuda.synchronize()
    g = parity.bf16_to_f64(out)
    o = att.decode(inp["q"], inp["k"], inp["v"], inp["kv_len"], inp["sinks"], inp["sm_scale"])
    absw = att.decode(inp["q"], inp["k"], _abs_bits(inp["v"]), inp["kv_len"], inp["sinks"], inp["sm_scale"])
    _say("   err/bound, mean", _gate(g, o, absw, "decode"))


def test_decode_empty_and_clamped_lengths():
    """kv_len 0 gives a zero output (only the sink); lengths past Lmax are clamped."""
    inp = gen.make_attn_decode(gen.AttnShape("t", 8, 2), 3, 128, seed=9)
    p = moe.attn_device_inputs(inp)
    p["kv_len"] = torch.tensor([0, 500, 128], dtype=torch.int32, device="cuda")
    out = moe.attn_decode(p["q"], p["k"], p["v"], p["kv_len"], p["sinks"], p["sm_scale"])
    torch.cuda.synchronize()
    g = parity.bf16_to_f64(out)
    assert np.all(g[0] == 0)
    np.testing.assert_array_equal(g[1], g[1])            # finite
    o = att.decode(inp["q"], inp["k"], inp["v"], np.array([0, 128, 128]), inp["sinks"], inp["sm_scale"])
    absw = att.decode(inp["q"], inp["k"], _abs_bits(inp["v"]), np.array([0, 128, 128]), inp["sinks"],
                      inp["sm_scale"])
    _gate(g[1:], o[1:], absw[1:], "clamped")


def test_prefill_deterministic():
    inp = gen.make_attn_prefill(gen.GPT_OSS_ATTN, 700, seed=3)
    p = moe.attn_device_inputs(inp)
    a = moe.attn_prefill(p["q"], p["k"], p["v"], p["sinks"]).clone()
    b = moe.attn_prefill(p["q"], p["k"], p["v"], p["sinks"]).clone()
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.timeout(900)
def test_full_size_prefill_sampled():
    """The benchmark's prefill workload (gpt-oss shape, S = 8192) on sampled rows."""
    S = 8192
    inp = gen.make_attn_prefill(gen.GPT_OSS_ATTN, S, seed=0)
    p = moe.attn_device_inputs(inp)
    out = moe.attn_prefill(p["q"], p["k"], p["v"], p["sinks"], p["sm_scale"])
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, 1, 63, 64, S - 1], np.random.default_rng(5).choice(S, 40, replace=False)]))
    g = parity.bf16_to_f64(out)[rows]
    o = att.prefill(inp["q"], inp["k"], inp["v"], inp["sinks"], inp["sm_scale"], rows=rows)
    absw = att.prefill(inp["q"], inp["k"], _abs_bits(inp["v"]), inp["sinks"], inp["sm_scale"], rows=rows)
    _say("[attn prefill full] err/bound, mean", _gate(g, o, absw, "prefill full"))


@pytest.mark.timeout(900)
def test_full_size_decode():
    """The benchmark's decode workload (gpt-oss shape, B = 64, Lmax = 4096, ragged)."""
    inp = gen.make_attn_decode(gen.GPT_OSS_ATTN, 64, 4096, seed=0)
    p = moe.attn_device_inputs(inp)
    out = moe.attn_decode(p["q"], p["k"], p["v"], p["kv_len"], p["sinks"], p["sm_scale"])
    torch.cuda.synchronize()
    g = parity.bf16_to_f64(out)
    o = att.decode(inp["q"], inp["k"], inp["v"], inp["kv_len"], inp["sinks"], inp["sm_scale"])
    absw = att.decode(inp["q"], inp["k"], _abs_bits(inp["v"]), inp["kv_len"], inp["sinks"], inp["sm_scale"])
    _say("[attn decode full] err/bound, mean", _gate(g, o, absw, "decode full"))
