"""Pins of the sink-attention oracle against things other than itself (CPU only).

A plausible slip (sink in the numerator, sink skipped, wrong GQA head map,
off-by-one causal mask, missing scale, transposed scores) fails one of them.
"""
import math

import numpy as np
import pytest
import torch

from oracle import attention as att
from oracle import codecs
from sparse_moe_layer_fp32_amd import inputs as gen

SH = gen.AttnShape("pins", 8, 2, 64)


def _sdpa(q, k, v, scale, causal):
    """torch's scaled_dot_product_attention in fp64, GQA by repeating kv heads.
    q [n_q, Hq, D], k/v [n_k, Hkv, D] -> [n_q, Hq, D]."""
    G = q.shape[1] // k.shape[1]
    tq = torch.from_numpy(q).permute(1, 0, 2)
    tk = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(G, 0)
    tv = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(G, 0)
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale)
    return o.permute(1, 0, 2).numpy()


def test_prefill_without_sink_is_causal_sdpa():
    p = gen.make_attn_prefill(SH, 37, seed=1)
    low = np.full(SH.Hq, -1e30, np.float32)
    o = att.prefill(p["q"], p["k"], p["v"], low, p["sm_scale"])
    ref = _sdpa(codecs.bf16_decode(p["q"]), codecs.bf16_decode(p["k"]), codecs.bf16_decode(p["v"]),
                p["sm_scale"], causal=True)
    np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-12)


def test_decode_without_sink_is_sdpa_over_the_cache():
    d = gen.make_attn_decode(SH, 4, 45, seed=2)
    low = np.full(SH.Hq, -1e30, np.float32)
    o = att.decode(d["q"], d["k"], d["v"], d["kv_len"], low, d["sm_scale"])
    for b in range(4):
        n = int(d["kv_len"][b])
        k = codecs.bf16_decode(d["k"][b, :, :n]).transpose(1, 0, 2)
        v = codecs.bf16_decode(d["v"][b, :, :n]).transpose(1, 0, 2)
        ref = _sdpa(codecs.bf16_decode(d["q"][b:b + 1]), k, v, d["sm_scale"], causal=False)
        np.testing.assert_allclose(o[b], ref[0], rtol=1e-12, atol=1e-12)


def test_first_position_closed_form():
    """Position 0 sees one key: o = v0 / (1 + exp(sink - s00))."""
    p = gen.make_attn_prefill(SH, 3, seed=3)
    o = att.prefill(p["q"], p["k"], p["v"], p["sinks"], p["sm_scale"])
    q, k, v = (codecs.bf16_decode(p[x]) for x in ("q", "k", "v"))
    for h in range(SH.Hq):
        kv = h // (SH.Hq // SH.Hkv)
        s = float(q[0, h] @ k[0, kv]) * p["sm_scale"]
        want = v[0, kv] / (1.0 + math.exp(float(p["sinks"][h]) - s))
        np.testing.assert_allclose(o[0, h], want, rtol=1e-13, atol=1e-15)


def test_large_sink_takes_all_the_mass():
    p = gen.make_attn_prefill(SH, 9, seed=4)
    o = att.prefill(p["q"], p["k"], p["v"], np.full(SH.Hq, 1e4, np.float32), p["sm_scale"])
    assert np.abs(o).max() < 1e-300


def test_brute_force_python_loops():
    """Pure-Python loops (math.exp, explicit GQA map and causal mask)."""
    sh = gen.AttnShape("tiny", 4, 2, 64)
    p = gen.make_attn_prefill(sh, 6, seed=5)
    o = att.prefill(p["q"], p["k"], p["v"], p["sinks"], p["sm_scale"])
    q, k, v = (codecs.bf16_decode(p[x]).tolist() for x in ("q", "k", "v"))
    for i in range(6):
        for h in range(4):
            kv = h // 2
            s = [sum(a * b for a, b in zip(q[i][h], k[j][kv])) * p["sm_scale"] for j in range(i + 1)]
            M = max([float(p["sinks"][h])] + s)
            w = [math.exp(x - M) for x in s]
            den = math.exp(float(p["sinks"][h]) - M) + sum(w)
            for dd in range(64):
                want = sum(w[j] * v[j][kv][dd] for j in range(i + 1)) / den
                assert abs(o[i, h, dd] - want) <= 1e-12 * (1 + abs(want))


def test_decode_is_key_permutation_invariant_and_matches_prefill_rows():
    p = gen.make_attn_prefill(SH, 20, seed=6)
    full = att.prefill(p["q"], p["k"], p["v"], p["sinks"], p["sm_scale"])
    i = 13
    kc = p["k"][:i + 1].transpose(1, 0, 2)[None]           # [1, Hkv, i+1, D]
    vc = p["v"][:i + 1].transpose(1, 0, 2)[None]
    o = att.decode(p["q"][i:i + 1], kc, vc, np.array([i + 1]), p["sinks"], p["sm_scale"])
    np.testing.assert_allclose(o[0], full[i], rtol=1e-13, atol=1e-15)
    perm = np.random.default_rng(7).permutation(i + 1)
    o2 = att.decode(p["q"][i:i + 1], kc[:, :, perm], vc[:, :, perm], np.array([i + 1]), p["sinks"], p["sm_scale"])
    np.testing.assert_allclose(o2, o, rtol=1e-13, atol=1e-15)


def test_sink_only_changes_the_normaliser():
    """Changing the sink rescales every output of a head by the same factor."""
    p = gen.make_attn_prefill(SH, 12, seed=8)
    a = att.prefill(p["q"], p["k"], p["v"], p["sinks"], p["sm_scale"])
    b = att.prefill(p["q"], p["k"], p["v"], p["sinks"] + np.float32(1.5), p["sm_scale"])
    ratio = b / np.where(a == 0, 1, a)
    for i in range(12):
        for h in range(SH.Hq):
            r = ratio[i, h]
            assert np.all(r < 1) and np.ptp(r) < 1e-9
