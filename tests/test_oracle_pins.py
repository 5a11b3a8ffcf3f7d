"""Pins of the CPU oracle against things other than itself (CPU only).

Each test names the part it pins. A plausible slip anywhere in the oracle
(a dropped bias, a swapped gate/up half, a wrong scale index, a transposed
operand, softmax over the wrong set, an unstable permutation) fails one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import codecs, oracle
from sparse_moe_layer_fp32_amd import inputs as gen
from tests import handworked

GOLD = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ------------------------------------------------------------------ P1: e4m3 decode
def test_e4m3_decode_format_points():
    fx = json.load(open(os.path.join(GOLD, "e4m3_points.json")))
    for code, val in fx["points"].items():
        got = codecs.E4M3_TABLE[int(code, 16)]
        assert got == val and math.copysign(1, got) == math.copysign(1, val), code
    for code in fx["nan_codes"]:
        assert np.isnan(codecs.E4M3_TABLE[int(code, 16)])
    assert np.sum(np.isnan(codecs.E4M3_TABLE)) == 2


def test_e4m3_decode_matches_torch_float8():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(codecs.E4M3_TABLE, ref)


# ------------------------------------------------------------------ P2: RNE encoder
def _brute_encode(v):
    """Nearest finite e4m3 value by exhaustive search; ties to the even code."""
    finite = [c for c in range(256) if not np.isnan(codecs.E4M3_TABLE[c])]
    best = None
    for c in finite:
        err = abs(codecs.E4M3_TABLE[c] - v)
        key = (err, c & 1)                      # tie -> even mantissa (lowest code bit 0)
        if best is None or key < best[0]:
            best = (key, c)
    c = best[1]
    if codecs.E4M3_TABLE[c] == 0:               # keep the sign of zero
        c = 0x80 if math.copysign(1, v) < 0 else 0x00
    return c


def test_e4m3_encoder_exhaustive_midpoints():
    pos = codecs.E4M3_TABLE[:0x7F]
    mids = (pos[:-1] + pos[1:]) / 2
    pts = np.concatenate([pos, mids, np.nextafter(mids.astype(np.float32), np.float32(0)),
                          np.nextafter(mids.astype(np.float32), np.float32(1e9)), [448.0]])
    pts = np.concatenate([pts, -pts]).astype(np.float32)
    got = codecs.e4m3_encode_rne(pts)
    want = np.array([_brute_encode(float(v)) for v in pts], np.uint8)
    np.testing.assert_array_equal(got, want)


def test_e4m3_encoder_random_vs_brute_and_torch():
    rng = np.random.default_rng(5)
    v = np.concatenate([rng.uniform(-448, 448, 2000), rng.normal(0, 1e-2, 2000),
                        rng.normal(0, 1, 2000)]).astype(np.float32)
    got = codecs.e4m3_encode_rne(v)
    want = np.array([_brute_encode(float(a)) for a in v[:1500]], np.uint8)
    np.testing.assert_array_equal(got[:1500], want)
    tq = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(got, tq)


def test_e4m3_encoder_saturates_and_nan():
    got = codecs.e4m3_encode_rne(np.array([460.0, -1e6, np.nan], np.float32))
    assert list(got) == [0x7E, 0xFE, 0x7F]


# ------------------------------------------------------------------ P3: router logits
def test_router_logits_vs_python_loops():
    rng = np.random.default_rng(1)
    T, d, E = 3, 7, 5
    x = gen.to_bf16_bits(rng.normal(size=(T, d)).astype(np.float32))
    W = rng.normal(size=(d, E)).astype(np.float32)
    b = rng.normal(size=E).astype(np.float32)
    got = oracle.router_logits(x, W, b)
    xf = gen.bf16_bits_to_f32(x)
    for t in range(T):
        for e in range(E):
            s = math.fsum(float(xf[t, i]) * float(W[i, e]) for i in range(d)) + float(b[e])
            assert abs(got[t, e] - s) <= 1e-14 * (1 + abs(s))


# ------------------------------------------------------------------ P4: top-k
def test_topk_is_the_k_largest_set_in_descending_order():
    rng = np.random.default_rng(2)
    L = rng.normal(size=(200, 12))
    L[0, :] = 1.0                                # all ties -> lowest indices
    for k in (1, 3, 12):
        idx = oracle.topk_select(L, k)
        for t in range(L.shape[0]):
            S = set(idx[t].tolist())
            rest = [e for e in range(12) if e not in S]
            assert len(S) == k
            if rest:
                assert min(L[t, list(S)]) >= max(L[t, rest])
            assert all(L[t, idx[t, j]] >= L[t, idx[t, j + 1]] for j in range(k - 1))
        assert list(idx[0]) == list(range(k))


# ------------------------------------------------------------------ P5: gate weights
def test_gate_weights_closed_forms():
    rng = np.random.default_rng(3)
    L = rng.normal(scale=3, size=(100, 8))
    w1 = oracle.gate_weights(L, oracle.topk_select(L, 1))
    assert np.all(w1 == 1.0)
    idx2 = oracle.topk_select(L, 2)
    w2 = oracle.gate_weights(L, idx2)
    l1 = np.take_along_axis(L, idx2, 1)
    logistic = 1.0 / (1.0 + np.exp(l1[:, 1] - l1[:, 0]))
    np.testing.assert_allclose(w2[:, 0], logistic, rtol=1e-14)
    idx4 = oracle.topk_select(L, 4)
    w4 = oracle.gate_weights(L, idx4)
    assert np.max(np.abs(w4.sum(1) - 1)) <= 1e-15
    assert np.all(np.diff(w4, axis=1) <= 0)       # ordered like the logits
    # softmax over the selected logits only: shifting an unselected logit changes nothing
    L2 = L.copy()
    for t in range(100):
        e = [x for x in range(8) if x not in idx4[t]][0]
        L2[t, e] -= 5.0
    np.testing.assert_array_equal(oracle.gate_weights(L2, idx4), w4)


# ------------------------------------------------------------------ P5b: routing variant and bf16 gate weights
def test_gate_weights_all_vs_library_softmax():
    """Softmax over all logits before top-k: the selected experts keep their
    full-softmax probabilities (scipy's softmax as the library special case)."""
    from scipy.special import softmax
    rng = np.random.default_rng(31)
    L = rng.normal(scale=2, size=(120, 16))
    for k in (1, 4, 16):
        idx = oracle.topk_select(L, k)
        w = oracle.gate_weights_all(L, idx)
        np.testing.assert_allclose(w, np.take_along_axis(softmax(L, axis=1), idx, 1), rtol=1e-13)
        assert np.all(np.diff(w, axis=1) <= 0)
        if k == 16:
            assert np.max(np.abs(w.sum(1) - 1)) <= 1e-14      # every expert selected: sums to 1
        else:
            assert np.all(w.sum(1) < 1)
    # unlike the selected-only softmax, an unselected logit moves the weights
    idx = oracle.topk_select(L, 4)
    L2 = L.copy()
    for t in range(len(L)):
        e = [x for x in range(16) if x not in idx[t]][0]
        L2[t, e] += 0.5
    assert not np.allclose(oracle.gate_weights_all(L2, idx), oracle.gate_weights_all(L, idx))
    # k = 1: the full softmax probability, a logistic against the log-sum-exp of the rest
    i1 = oracle.topk_select(L, 1)
    l_top = np.take_along_axis(L, i1, 1)[:, 0]
    others = np.log(np.exp(L).sum(1) - np.exp(l_top))
    np.testing.assert_allclose(oracle.gate_weights_all(L, i1)[:, 0],
                               1.0 / (1.0 + np.exp(others - l_top)), rtol=1e-12)


def test_bf16_gate_weights():
    rng = np.random.default_rng(32)
    w = rng.uniform(0, 1, size=5000)
    r = oracle.bf16_round_weights(w)
    # every value is a bf16 (via torch's exact bf16 cast of the rounded value) and is the nearest one
    np.testing.assert_array_equal(torch.from_numpy(r).to(torch.bfloat16).to(torch.float64).numpy(), r)
    np.testing.assert_array_equal(r, torch.from_numpy(w).to(torch.bfloat16).to(torch.float64).numpy())
    assert np.all(np.abs(r - w) <= 2.0 ** -8 * np.abs(w))      # 8 significant bits: unit roundoff 2^-8


def test_route_options_change_only_the_weights():
    layer = gen.custom_layer(256, 256, 8, 3, layer_id=333)
    inp = gen.make_inputs(layer, T=50)
    a = oracle.route(inp)
    b = oracle.route(dict(inp, routing="softmax_topk"))
    c = oracle.route(dict(inp, routing="softmax_topk", gate_bf16=True))
    for key in ("idx", "counts", "offsets", "row_of", "row_token"):
        np.testing.assert_array_equal(a[key], b[key])
        np.testing.assert_array_equal(a[key], c[key])
    # the selected-only weights are the all-expert ones renormalised over the k
    np.testing.assert_allclose(a["w"], b["w"] / b["w"].sum(1, keepdims=True), rtol=1e-13)
    np.testing.assert_array_equal(c["w"], oracle.bf16_round_weights(b["w"]))
    with pytest.raises(ValueError):
        oracle.route(dict(inp, routing="bogus"))


# ------------------------------------------------------------------ P6: permutation
@pytest.mark.parametrize("T,E,k", [(1, 4, 2), (37, 8, 3), (300, 64, 8), (5, 3, 3)])
def test_permutation_invariants(T, E, k):
    rng = np.random.default_rng(T * E + k)
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    counts, offsets, row_of, row_token = oracle.permutation(idx, E)
    np.testing.assert_array_equal(counts, np.bincount(idx.ravel(), minlength=E))
    assert offsets[0] == 0 and np.all(np.diff(offsets) == counts) and offsets[-1] == T * k
    assert sorted(row_of.ravel().tolist()) == list(range(T * k))     # bijection
    for t in range(T):
        for j in range(k):
            r = row_of[t, j]
            e = idx[t, j]
            assert offsets[e] <= r < offsets[e + 1]
            assert row_token[r] == t
    for e in range(E):                                                 # stable in token order
        toks = row_token[offsets[e]:offsets[e + 1]]
        assert np.all(np.diff(toks) > 0)


# ------------------------------------------------------------------ P7: activation quantisation
def test_quantize_groups_properties():
    rng = np.random.default_rng(4)
    v = (rng.normal(size=(40, 512)) * rng.uniform(0.01, 10, size=(40, 1))).astype(np.float32)
    v[3, 128:256] = 0.0                                  # an all-zero group
    q, s = oracle.quantize_groups(v)
    assert s.dtype == np.float32 and s.shape == (40, 4)
    assert s[3, 1] == 1.0 and np.all(q[3, 128:256] == 0)
    vals = codecs.e4m3_decode(q)
    assert np.all(np.abs(vals) <= 448)
    g = v.reshape(40, 4, 128)
    am = np.abs(g).argmax(axis=2)
    for r in range(40):
        for c in range(4):
            if r == 3 and c == 1:
                continue
            a = g[r, c, am[r, c]]
            assert vals.reshape(40, 4, 128)[r, c, am[r, c]] == math.copysign(448, a)
    deq = oracle.dequant_groups(q, s)
    # error at most half an e4m3 spacing (relative 2^-4 for normals, 2^-10 * s absolute below)
    err = np.abs(deq - v)
    bound = np.maximum(np.abs(v) * 2.0 ** -4, np.repeat(s, 128, axis=1) * 2.0 ** -10)
    assert np.all(err <= bound * (1 + 1e-6))
    q2, s2 = oracle.quantize_groups(deq.astype(np.float32))
    np.testing.assert_array_equal(codecs.e4m3_decode(q2) * np.repeat(s2, 128, 1), deq)


def test_quantize_groups_vs_torch_cast():
    """Special case reducing to a library routine: scale by fl32(amax/448), then
    PyTorch's float8_e4m3fn cast (round-to-nearest-even)."""
    rng = np.random.default_rng(6)
    v = rng.normal(size=(64, 384)).astype(np.float32)
    q, s = oracle.quantize_groups(v)
    t = torch.from_numpy(v).view(64, 3, 128)
    ts = t.abs().amax(dim=2, keepdim=True) / 448.0
    tq = (t / ts).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8).reshape(64, 384)
    np.testing.assert_array_equal(q, tq.numpy())
    np.testing.assert_array_equal(s, ts.squeeze(2).numpy())


# ------------------------------------------------------------------ P8: k=1, E=1 -> dense biased SwiGLU MLP
def _torch_quant(v32):
    n, K = v32.shape
    g = v32.view(n, K // 128, 128)
    am = g.abs().amax(dim=2, keepdim=True)
    s = torch.where(am > 0, am / 448.0, torch.ones_like(am))
    q = (g / s).clamp(-448, 448).to(torch.float8_e4m3fn).to(torch.float64)
    return (q * s.double()).view(n, K)


def _torch_weight(codes, scales):
    K, N = codes.shape
    w = torch.from_numpy(codes).view(torch.float8_e4m3fn).double()
    s = torch.from_numpy(scales).double().repeat_interleave(128, 0).repeat_interleave(128, 1)
    return w * s


def test_single_expert_reduces_to_dense_swiglu_mlp():
    layer = gen.custom_layer(256, 384, 1, 1, d_real=200, layer_id=201)
    inp = gen.make_inputs(layer, T=24)
    res = oracle.forward(inp)
    bf = lambda b: torch.from_numpy(gen.bf16_bits_to_f32(b)).double()
    x = bf(inp["x"]).float()
    f = inp["f"]
    P = _torch_quant(x) @ _torch_weight(inp["W_gateup"][0], inp["S_gateup"][0]) + bf(inp["b_gateup"][0])
    h = torch.nn.functional.silu(P[:, :f]) * P[:, f:]
    dense = _torch_quant(h.float()) @ _torch_weight(inp["W_down"][0], inp["S_down"][0]) + bf(inp["b_down"][0])
    np.testing.assert_allclose(res["out64"], dense.numpy(), rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------------ P9: sparse routing vs all-experts brute force
@pytest.mark.parametrize("T,d,f,E,k", [(8, 128, 128, 4, 2), (64, 256, 256, 8, 2), (9, 256, 128, 6, 6)])
def test_sparse_block_equals_all_experts_brute_force(T, d, f, E, k):
    layer = gen.custom_layer(d, f, E, k, layer_id=300 + E)
    inp = gen.make_inputs(layer, T=T)
    res = oracle.forward(inp)
    xf = gen.bf16_bits_to_f32(inp["x"]).astype(np.float64)
    L = xf @ inp["W_router"].astype(np.float64) + inp["b_router"].astype(np.float64)
    xdeq = oracle.dequant_groups(*oracle.quantize_groups(xf.astype(np.float32)))
    out = np.zeros((T, d))
    for t in range(T):
        for e in range(E):
            rank = sum(1 for e2 in range(E) if L[t, e2] > L[t, e] or (L[t, e2] == L[t, e] and e2 < e))
            if rank >= k:
                continue
            sel = [e2 for e2 in range(E)
                   if sum(1 for e3 in range(E) if L[t, e3] > L[t, e2] or (L[t, e3] == L[t, e2] and e3 < e2)) < k]
            w = math.exp(L[t, e]) / sum(math.exp(L[t, e2]) for e2 in sel)
            Y = oracle.expert_mlp(xdeq[t:t + 1], inp["W_gateup"][e], inp["S_gateup"][e], inp["b_gateup"][e],
                                  inp["W_down"][e], inp["S_down"][e], inp["b_down"][e])
            out[t] += w * Y[0]
    np.testing.assert_allclose(res["out64"], out, rtol=1e-12, atol=1e-12 * np.abs(out).max())


# ------------------------------------------------------------------ P10: padding
def test_padded_columns_are_exactly_zero():
    layer = gen.custom_layer(384, 256, 6, 2, d_real=300, layer_id=401)
    inp = gen.make_inputs(layer, T=20)
    res = oracle.forward(inp)
    assert np.all(res["out64"][:, 300:] == 0.0)
    assert np.abs(res["out64"][:, :300]).min() > 0


# ------------------------------------------------------------------ P11: token independence
def test_token_independence():
    inp = gen.make_inputs("c0")
    full = oracle.forward(inp)["out64"]
    sub = [5, 0, 63, 17]
    part = oracle.forward(inp, tokens=sub)["out64"]
    np.testing.assert_allclose(part, full[sub], rtol=1e-13, atol=1e-13)
    perm = np.random.default_rng(7).permutation(inp["T"])
    inp2 = dict(inp, x=inp["x"][perm])
    np.testing.assert_allclose(oracle.forward(inp2)["out64"], full[perm], rtol=1e-13, atol=1e-13)
    inp3 = dict(inp, x=inp["x"][:10], T=10)
    np.testing.assert_allclose(oracle.forward(inp3)["out64"], full[:10], rtol=1e-13, atol=1e-13)


# ------------------------------------------------------------------ hand-worked block (closed forms)
@pytest.mark.parametrize("k", [1, 2])
def test_handworked_block(k):
    inp = handworked.build(k)
    res = oracle.forward(inp)
    want = handworked.expected(k)
    assert list(res["idx"][0]) == ([0] if k == 1 else [0, 1])
    np.testing.assert_allclose(res["out64"][0], want, rtol=0, atol=1e-6 * np.abs(want).max())
    assert res["xq"][0, 0] == 0x7E and res["xq"][0, 1] == 0x76 and res["xs"][0, 0] == 2.0 ** -7


# ------------------------------------------------------------------ SwiGLU form
def test_silu_vs_torch():
    z = np.linspace(-60, 60, 2001)
    np.testing.assert_allclose(oracle.silu(z), torch.nn.functional.silu(torch.from_numpy(z)).numpy(),
                               rtol=1e-15, atol=1e-300)


# ------------------------------------------------------------------ MXFP8 variant
def test_e8m0_decode_format_points():
    fx = json.load(open(os.path.join(GOLD, "e8m0_points.json")))
    for code, val in fx["points"].items():
        assert codecs.e8m0_decode(np.uint8(int(code, 16))) == val, code
    for code in fx["nan_codes"]:
        assert np.isnan(codecs.e8m0_decode(np.uint8(int(code, 16))))
    allv = codecs.e8m0_decode(np.arange(255, dtype=np.uint8))
    assert np.all(allv[1:] == 2 * allv[:-1])                 # consecutive powers of two


def _mx_exponent_frexp(a):
    """Independent derivation: a = m 2^p, m in [0.5, 1); 448 = 0.875 * 2^9."""
    m, p = np.frexp(np.asarray(a, np.float64))
    e = np.where(m <= 0.875, p - 9, p - 8)
    return np.clip(np.where(a > 0, e, -127), -127, 127)


def test_mx_scale_exponent_closed_forms_and_minimality():
    f32 = np.float32
    cases = {448.0: 0, 3.5: -7, 1.0: -8, 0.875: -9, 0.0: -127, 449.0: 1, 224.0: -1, 224.5: 0,
             float(np.nextafter(f32(448), f32(1e9))): 1, float(np.nextafter(f32(448), f32(0))): 0,
             448.0 * 2.0 ** 100: 100, 448.0 * 2.0 ** -126: -126, 1e-45: -127}
    for a, e in cases.items():
        assert int(oracle.mx_scale_exponent(np.array(a))) == e, a
    rng = np.random.default_rng(11)
    a = np.concatenate([
        np.abs(rng.normal(size=4000) * np.exp(rng.uniform(-60, 60, 4000))),
        # ulp neighbours of 448 * 2^n, where a rounding slip would show
        np.nextafter(np.float32(448) * np.float32(2.0) ** np.arange(-40, 40, dtype=np.float32),
                     np.float32(np.inf)),
        np.nextafter(np.float32(448) * np.float32(2.0) ** np.arange(-40, 40, dtype=np.float32),
                     np.float32(0)),
    ]).astype(np.float32).astype(np.float64)
    e = oracle.mx_scale_exponent(a)
    assert np.all(a <= 448.0 * np.ldexp(1.0, e))
    assert np.all((e == -127) | (a > 448.0 * np.ldexp(1.0, e - 1)))
    np.testing.assert_array_equal(e, _mx_exponent_frexp(a))


def test_quantize_mx_vs_torch_cast():
    """Library special case: the power-of-two scale from the frexp derivation,
    then PyTorch's float8_e4m3fn cast of v / 2^e (exact division)."""
    rng = np.random.default_rng(12)
    v = (rng.normal(size=(48, 256)) * np.exp(rng.uniform(-8, 8, size=(48, 8))).repeat(32, 1))
    v = v.astype(np.float32)
    v[5, 64:96] = 0.0
    q, sc = oracle.quantize_mx(v)
    t = torch.from_numpy(v).double().view(48, 8, 32)
    e = torch.from_numpy(_mx_exponent_frexp(t.abs().amax(dim=2).numpy()))
    tq = (t / torch.ldexp(torch.ones(()), e.double()).unsqueeze(2)).float()
    tq = tq.to(torch.float8_e4m3fn).view(torch.uint8).reshape(48, 256).numpy()
    np.testing.assert_array_equal(q, tq)
    np.testing.assert_array_equal(sc, (e.numpy() + 127).astype(np.uint8))
    assert sc[5, 2] == 0 and np.all(q[5, 64:96] == 0)


def test_quantize_mx_properties():
    rng = np.random.default_rng(13)
    v = (rng.normal(size=(30, 128)) * rng.uniform(1e-3, 1e3, size=(30, 1))).astype(np.float32)
    q, sc = oracle.quantize_mx(v)
    assert q.shape == (30, 128) and sc.shape == (30, 4) and sc.dtype == np.uint8
    vals = codecs.e4m3_decode(q).reshape(30, 4, 32)
    # amax / 2^e lies in (224, 448] (the scale is as small as it can be), so
    # the block's largest code is in [224, 448] (e4m3 rounds (224, 232] to 224)
    bmax = np.abs(vals).max(axis=2)
    assert np.all(bmax >= 224) and np.all(bmax <= 448)
    deq = oracle.dequant_mx(q, sc)
    X = np.repeat(codecs.e8m0_decode(sc), 32, axis=1)
    err = np.abs(deq - v)
    assert np.all(err <= np.maximum(np.abs(v) * 2.0 ** -4, X * 2.0 ** -10) * (1 + 1e-12))
    # its own output is a fixed point in value (a block whose max rounded down
    # to 224 X re-quantises with X / 2 and doubled codes)
    q2, sc2 = oracle.quantize_mx(deq.astype(np.float32))
    np.testing.assert_array_equal(oracle.dequant_mx(q2, sc2), deq)
    # blocks are independent: scaling one block by 2^5 moves only its scale
    v3 = v.copy()
    v3[:, 32:64] *= np.float32(32.0)
    q3, sc3 = oracle.quantize_mx(v3)
    np.testing.assert_array_equal(q3, q)
    np.testing.assert_array_equal(sc3[:, 1], sc[:, 1] + 5)
    np.testing.assert_array_equal(np.delete(sc3, 1, axis=1), np.delete(sc, 1, axis=1))


def test_dequant_weight_mx_brute_force_and_block_reduction():
    rng = np.random.default_rng(14)
    K, N = 256, 384
    codes = rng.integers(0, 256, size=(K, N), dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x3A
    sc = rng.integers(100, 150, size=(K // 32, N), dtype=np.uint8)
    W = oracle.dequant_weight_mx(codes, sc)
    for (kk, n) in [(0, 0), (31, 5), (32, 5), (255, 383), (100, 200), (64, 130)]:
        assert W[kk, n] == codecs.E4M3_TABLE[codes[kk, n]] * 2.0 ** (int(sc[kk // 32, n]) - 127)
    # scales constant over each 128x128 block: the 128x128 block-scaled format
    blk = rng.integers(110, 140, size=(K // 128, N // 128))
    sc_mx = np.repeat(np.repeat(blk, 4, axis=0), 128, axis=1).astype(np.uint8)
    S = np.ldexp(1.0, blk - 127).astype(np.float32)
    np.testing.assert_array_equal(oracle.dequant_weight_mx(codes, sc_mx), oracle.dequant_weight(codes, S))


def test_mx_weight_conversion_round_trip():
    """The generator's static MX conversion, checked against the oracle's MX
    quantiser applied along K (the same rule, written independently)."""
    rng = np.random.default_rng(15)
    w = (rng.normal(size=(128, 256)) * 0.05).astype(np.float32)
    w[:32, 7] = 0.0
    codes, sc = gen.quantize_weight_mx(w)
    q, s = oracle.quantize_mx(np.ascontiguousarray(w.T))
    np.testing.assert_array_equal(codes, q.T)
    np.testing.assert_array_equal(sc, s.T)


def _torch_quant_mx(v32):
    n, K = v32.shape
    g = v32.double().view(n, K // 32, 32)
    e = torch.from_numpy(_mx_exponent_frexp(g.abs().amax(dim=2).numpy())).double()
    X = torch.ldexp(torch.ones(()), e).unsqueeze(2)
    q = (g / X).float().to(torch.float8_e4m3fn).double()
    return (q * X).view(n, K)


def test_mx_single_expert_reduces_to_dense_swiglu_mlp():
    layer = gen.custom_layer(256, 384, 1, 1, d_real=200, layer_id=202)
    inp = gen.make_inputs(layer, T=24, fmt="mx")
    res = oracle.forward(inp)
    bf = lambda b: torch.from_numpy(gen.bf16_bits_to_f32(b)).double()
    x = bf(inp["x"]).float()
    f = inp["f"]

    def wdeq(codes, sc):
        w = torch.from_numpy(codes).view(torch.float8_e4m3fn).double()
        return w * torch.ldexp(torch.ones(()), torch.from_numpy(sc.astype(np.int64) - 127).double()
                               ).repeat_interleave(32, 0)

    P = _torch_quant_mx(x) @ wdeq(inp["W_gateup"][0], inp["S_gateup"][0]) + bf(inp["b_gateup"][0])
    h = torch.nn.functional.silu(P[:, :f]) * P[:, f:]
    dense = _torch_quant_mx(h.float()) @ wdeq(inp["W_down"][0], inp["S_down"][0]) + bf(inp["b_down"][0])
    np.testing.assert_allclose(res["out64"], dense.numpy(), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("T,d,f,E,k", [(8, 128, 128, 4, 2), (9, 256, 128, 6, 6)])
def test_mx_sparse_block_equals_all_experts_brute_force(T, d, f, E, k):
    layer = gen.custom_layer(d, f, E, k, layer_id=320 + E)
    inp = gen.make_inputs(layer, T=T, fmt="mx")
    res = oracle.forward(inp)
    xf = gen.bf16_bits_to_f32(inp["x"]).astype(np.float64)
    L = xf @ inp["W_router"].astype(np.float64) + inp["b_router"].astype(np.float64)
    xdeq = _torch_quant_mx(torch.from_numpy(xf.astype(np.float32))).numpy()
    out = np.zeros((T, d))
    for t in range(T):
        rank = lambda e: sum(1 for e2 in range(E) if L[t, e2] > L[t, e] or (L[t, e2] == L[t, e] and e2 < e))
        sel = [e for e in range(E) if rank(e) < k]
        for e in sel:
            w = math.exp(L[t, e]) / sum(math.exp(L[t, e2]) for e2 in sel)
            Y = oracle.expert_mlp(xdeq[t:t + 1], inp["W_gateup"][e], inp["S_gateup"][e], inp["b_gateup"][e],
                                  inp["W_down"][e], inp["S_down"][e], inp["b_down"][e], fmt="mx")
            out[t] += w * Y[0]
    np.testing.assert_allclose(res["out64"], out, rtol=1e-12, atol=1e-12 * np.abs(out).max())


@pytest.mark.parametrize("k", [1, 2])
def test_handworked_block_mx(k):
    inp = handworked.build(k, fmt="mx")
    res = oracle.forward(inp)
    want = handworked.expected(k, fmt="mx")
    assert list(res["idx"][0]) == ([0] if k == 1 else [0, 1])
    np.testing.assert_allclose(res["out64"][0], want, rtol=0, atol=1e-12 * np.abs(want).max())
    assert res["xq"][0, 0] == 0x7E and res["xq"][0, 1] == 0x76 and res["xs"][0, 0] == 127 - 7


# ------------------------------------------------------------------ MXFP4 weights
def test_e2m1_decode_format_points():
    fx = json.load(open(os.path.join(GOLD, "e2m1_points.json")))
    for code, val in fx["points"].items():
        got = codecs.E2M1_TABLE[int(code, 16)]
        assert got == val and math.copysign(1, got) == math.copysign(1, val), code
    # every E2M1 value is an e4m3 value (the reduction the pins below rely on)
    assert np.all(np.isin(codecs.E2M1_TABLE, codecs.E4M3_TABLE))


def _brute_e2m1(v):
    """Nearest E2M1 code by exhaustive search over the 8 magnitudes; a tie goes
    to the even code (mantissa bit 0); the sign bit follows v."""
    a = min(abs(v), 6.0)
    best = min(range(8), key=lambda c: (abs(codecs.E2M1_TABLE[c] - a), c % 2))
    return best | (8 if math.copysign(1, v) < 0 else 0)


def test_e2m1_encoder_vs_brute_force():
    mags = codecs.E2M1_TABLE[:8]
    mids = (mags[1:] + mags[:-1]) / 2
    vals = np.concatenate([mags, mids, np.nextafter(mids, 0), np.nextafter(mids, 10), [6.5, 100.0, 1e-9],
                           np.random.default_rng(16).uniform(0, 7, 500)])
    vals = np.concatenate([vals, -vals])
    got = codecs.e2m1_encode_rne(vals)
    want = np.array([_brute_e2m1(float(v)) for v in vals], np.uint8)
    np.testing.assert_array_equal(got, want)


def test_unpack_fp4_order():
    packed = np.array([[0x42, 0x09], [0xF1, 0x70]], np.uint8)      # [K/2 = 2, N = 2]
    codes = codecs.unpack_fp4_k(packed)
    np.testing.assert_array_equal(codes, [[0x2, 0x9], [0x4, 0x0], [0x1, 0x0], [0xF, 0x7]])


def _fp4_as_mx(packed, scales):
    """The same weights as MX e4m3 codes (exact: every E2M1 value is an e4m3 value)."""
    vals = codecs.e2m1_decode(codecs.unpack_fp4_k(packed))
    return codecs.e4m3_encode_rne(vals), scales


def test_dequant_weight_mxfp4_reduces_to_mx():
    rng = np.random.default_rng(17)
    packed = rng.integers(0, 256, size=(64, 256), dtype=np.uint8)    # K = 128
    sc = rng.integers(110, 140, size=(4, 256), dtype=np.uint8)
    W = oracle.dequant_weight_mxfp4(packed, sc)
    np.testing.assert_array_equal(W, oracle.dequant_weight_mx(*_fp4_as_mx(packed, sc)))
    assert W[1, 0] == codecs.E2M1_TABLE[packed[0, 0] >> 4] * 2.0 ** (int(sc[0, 0]) - 127)
    assert W[33, 7] == codecs.E2M1_TABLE[packed[16, 7] >> 4] * 2.0 ** (int(sc[1, 7]) - 127)


def test_mxfp4_weight_conversion_vs_oracle_codec():
    """The generator's static MXFP4 conversion against the oracle's E2M1 encoder
    with the scale found by search: the smallest 2^e with amax <= 6 * 2^e."""
    rng = np.random.default_rng(18)
    w = (rng.normal(size=(128, 64)) * 0.05).astype(np.float32)
    w[32:64, 3] = 0.0
    packed, sc = gen.quantize_weight_mxfp4(w)
    for b in range(4):
        for n in range(64):
            blk = w[32 * b:32 * b + 32, n].astype(np.float64)
            am = np.abs(blk).max()
            e = next(e for e in range(-127, 128) if am <= 6.0 * 2.0 ** e)
            assert sc[b, n] == e + 127, (b, n)
            codes = codecs.e2m1_encode_rne(blk / 2.0 ** e)
            np.testing.assert_array_equal(codecs.unpack_fp4_k(packed)[32 * b:32 * b + 32, n], codes)


def test_mxfp4_forward_equals_mx_with_the_same_weights():
    layer = gen.custom_layer(256, 128, 5, 2, layer_id=330)
    inp = gen.make_inputs(layer, T=20, fmt="mxfp4")
    mx = dict(inp, format="mx")
    for key in ("W_gateup", "W_down"):
        mx[key] = np.stack([_fp4_as_mx(inp[key][e], None)[0] for e in range(inp["E"])])
    a, b = oracle.forward(inp)["out64"], oracle.forward(mx)["out64"]
    np.testing.assert_array_equal(a, b)


@pytest.mark.parametrize("k", [1, 2])
def test_handworked_block_mxfp4(k):
    inp = handworked.build(k, fmt="mxfp4")
    assert inp["W_gateup"].shape == (2, 64, 256) and inp["W_gateup"][0, 0, 0] == 0x42
    res = oracle.forward(inp)
    want = handworked.expected(k, fmt="mxfp4")
    np.testing.assert_allclose(res["out64"][0], want, rtol=0, atol=1e-12 * np.abs(want).max())
