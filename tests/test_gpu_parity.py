"""HIP path vs the CPU oracle, element by element, through the C ABI (GPU only).

Small cases run the oracle on every token and cover both GEMM paths (large
row tiles and small row tiles) and the three weight formats (128x128
block-scaled FP8, MXFP8, MXFP4), ragged expert tails, padded hidden sizes, column tails, k = 1,
k = E and E = 256, k = 8.  Full-size workloads check the
routing, permutation and x quantisation on every token and the expert rows
and outputs on a seeded sample of tokens, in the launch configuration the
benchmark times.  Gates are those of ``tests/parity.py``.
"""
import sys

import numpy as np
import pytest
import torch

import sparse_moe_layer_fp32_amd as moe
from sparse_moe_layer_fp32_amd import inputs as gen
from tests import handworked, parity

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def run_debug(inp, path):
    p = moe.device_inputs(inp)
    dbg = moe.forward_debug(p["x"], p["W_router"], p["b_router"], p["k"], p["W_gateup"],
                            p["S_gateup"], p["b_gateup"], p["W_down"], p["S_down"], p["b_down"],
                            path=path, routing=inp.get("routing", "topk_softmax"),
                            gate_bf16=inp.get("gate_bf16", False), fmt=p["fmt"])
    torch.cuda.synchronize()
    return dbg


FMTS = ["block128", "mx", "mxfp4"]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("path", ["prefill", "decode"])
@pytest.mark.parametrize("k", [1, 2])
def test_handworked_block(k, path, fmt):
    inp = handworked.build(k, fmt=fmt)
    _say(f"[handworked] k={k} path={path} fmt={fmt}")
    dbg = run_debug(inp, path)
    g = parity.bf16_to_f64(dbg["out"])[0]
    want = handworked.expected(k, fmt=fmt)
    # bf16 output of a hand-derived value: within one bf16 half-spacing (2^-9 relative) + h rounding
    np.testing.assert_allclose(g, want, rtol=2.0 ** -8, atol=1e-6)
    assert sorted(dbg["topk_idx"].cpu().numpy()[0].tolist()) == ([0] if k == 1 else [0, 1])
    xq = dbg["xq"].cpu().numpy()[0]
    assert xq[0] == 0x7E and xq[1] == 0x76 and np.all(xq[2:] == 0)
    xs = dbg["xs"].cpu().numpy()[0]
    if fmt != "block128":
        assert xs[0] == 127 - 7 and np.all(xs[1:] == 0)       # 2^-7, then all-zero blocks
    else:
        assert xs[0] == 2.0 ** -7


SMALL = [
    # (T, d, d_real, f, E, k)
    (64, 256, 256, 256, 8, 2),          # the tiny config
    (1, 128, 128, 128, 2, 1),           # one token
    (37, 384, 300, 256, 6, 3),          # ragged T, padded hidden size
    (1000, 256, 256, 256, 4, 2),        # ~500 rows per expert: several row tiles + tails
    (77, 128, 128, 128, 256, 8),        # E = 256, k = 8
    (50, 256, 256, 128, 5, 5),          # k = E (every expert)
    (130, 640, 640, 384, 3, 1),         # k = 1, down-projection column tail (640 = 2.5 x 256)
    (513, 384, 384, 512, 7, 3),         # odd expert count, T not a multiple of 16
    (2100, 384, 384, 256, 20, 2),       # 128-token router workgroups, 3 K splits, ragged last block
    (2048, 256, 256, 128, 128, 4),      # 128-token router workgroups with E = 128
    (32800, 128, 128, 128, 8, 1),       # 128-token router workgroups, one split: top-k in the router
]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("path", ["prefill", "decode"])
@pytest.mark.parametrize("shape", SMALL, ids=[f"T{s[0]}-d{s[1]}-f{s[3]}-E{s[4]}-k{s[5]}" for s in SMALL])
def test_small_shapes_vs_oracle(shape, path, fmt):
    T, d, dr, f, E, k = shape
    layer = gen.custom_layer(d, f, E, k, d_real=dr, layer_id=1000 + d + f + E + k)
    inp = gen.make_inputs(layer, T=T, fmt=fmt)
    _say(f"[small] shape={shape} path={path} fmt={fmt}")
    dbg = run_debug(inp, path)
    ref = parity.oracle_ref(inp)
    parity.check_routing(dbg, ref, T, k)
    parity.check_xquant(dbg, ref["xq"], ref["xs"])
    nflip, ncodes = parity.check_h_decisions(dbg, ref, fmt)
    worst = parity.check_down_stage(dbg, ref, inp, dr)
    parity.check_combine_stage(dbg)
    g = parity.bf16_to_f64(dbg["out"])
    m = parity.check_end_to_end(g, dbg, ref, inp, dr)
    assert np.all(g[:, dr:] == 0), "padded output columns must be exactly zero"
    _say(f"   out {m}\n   h decisions differing from the oracle: {nflip}/{ncodes}; "
         f"down-stage err/bound {worst:.3f}")


@pytest.mark.parametrize("d,f", [(768, 512), (384, 384)])
@pytest.mark.parametrize("fmt", FMTS)
def test_tile_counter_schedule_vs_oracle(fmt, d, f):
    """Prefill GEMMs whose tile lists outgrow the static first two tiles of
    every workgroup (2 x 256), with at least 3 K blocks per tile: the rest is
    handed out by the per-XCD tile counters, inside XCD ranges of equal cost.
    A Zipf-skewed 256-expert layer gives about 270 row blocks, most of them
    short.  With d = 768, f = 512 the gate/up GEMM has 6 K blocks and the down
    GEMM 4; with d = f = 384 both have 3, the fewest the counters serve, where
    the index fetched for a tile is stored one step after the atomic and read
    in the next (and the down GEMM's last column tile is half wide).  Every
    token against the oracle: a tile computed twice or never would show."""
    layer = gen.custom_layer(d, f, 256, 8, layer_id=7000, router="zipf")
    inp = gen.make_inputs(layer, T=1024, fmt=fmt)
    ref = parity.oracle_ref(inp)
    rows = np.diff(ref["offsets"])
    blocks = int(sum(-(-int(c) // 192) for c in rows))
    assert blocks * (f // 128) > 512 and blocks * -(-d // 256) > 512, blocks
    _say(f"[schedule] fmt={fmt} d={d} f={f} row blocks {blocks}")
    dbg = run_debug(inp, "prefill")
    parity.check_routing(dbg, ref, inp["T"], inp["k"])
    parity.check_xquant(dbg, ref["xq"], ref["xs"])
    nflip, ncodes = parity.check_h_decisions(dbg, ref, fmt)
    worst = parity.check_down_stage(dbg, ref, inp, inp["d_real"])
    parity.check_combine_stage(dbg)
    g = parity.bf16_to_f64(dbg["out"])
    m = parity.check_end_to_end(g, dbg, ref, inp, inp["d_real"])
    _say(f"   out {m}\n   h flips {nflip}/{ncodes}; down-stage err/bound {worst:.3f}")


# Decode batches with fewer GEMM tiles than the chip's workgroup slots: both
# decode GEMMs cut every tile into K ranges (split K), write fp32 partial sums
# and a finish kernel adds them in split order before the epilogue.
# (T, d, d_real, f, E, k) and the (gate/up, down) split counts they get.
SPLITK = [
    (1, 1024, 1024, 1024, 8, 2),        # splits 2, 2
    (3, 2048, 2000, 1024, 16, 4),       # splits 4, 2; padded hidden size
    (5, 1536, 1536, 1536, 64, 4),       # splits 2, 2
]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("shape", SPLITK, ids=[f"T{s[0]}-d{s[1]}-f{s[3]}-E{s[4]}-k{s[5]}" for s in SPLITK])
def test_split_k_decode_vs_oracle(shape, fmt):
    T, d, dr, f, E, k = shape
    layer = gen.custom_layer(d, f, E, k, d_real=dr, layer_id=6000 + d + f + E + k)
    inp = gen.make_inputs(layer, T=T, fmt=fmt)
    _say(f"[splitk] shape={shape} fmt={fmt}")
    dbg = run_debug(inp, "decode")
    ref = parity.oracle_ref(inp)
    parity.check_routing(dbg, ref, T, k)
    parity.check_xquant(dbg, ref["xq"], ref["xs"])
    nflip, ncodes = parity.check_h_decisions(dbg, ref, fmt)
    worst = parity.check_down_stage(dbg, ref, inp, dr)
    parity.check_combine_stage(dbg)
    g = parity.bf16_to_f64(dbg["out"])
    m = parity.check_end_to_end(g, dbg, ref, inp, dr)
    assert np.all(g[:, dr:] == 0)
    _say(f"   out {m}\n   h flips {nflip}/{ncodes}; down-stage err/bound {worst:.3f}")


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("cfg,T", [("c1", 1), ("c1", 2), ("c4a", 1)])
def test_split_k_full_layers(cfg, T, fmt):
    """The gpt-oss-20b-like and the 128-expert layers at one and two tokens
    (split K on both GEMMs), every token against the oracle, and repeat calls
    bit-identical."""
    inp = gen.make_inputs(cfg, T=T, fmt=fmt)
    _say(f"[splitk] {cfg} T={T} fmt={fmt}")
    dbg = run_debug(inp, "auto")
    ref = parity.oracle_ref(inp)
    dr = inp["d_real"]
    parity.check_routing(dbg, ref, T, inp["k"])
    parity.check_xquant(dbg, ref["xq"], ref["xs"])
    parity.check_h_decisions(dbg, ref, fmt)
    parity.check_down_stage(dbg, ref, inp, dr)
    parity.check_combine_stage(dbg)
    g = parity.bf16_to_f64(dbg["out"])
    m = parity.check_end_to_end(g, dbg, ref, inp, dr)
    assert np.all(g[:, dr:] == 0)
    again = parity.bf16_to_f64(run_debug(inp, "auto")["out"])
    np.testing.assert_array_equal(again, g)
    _say(f"   out {m}")
    parity.record(dict(cfg=f"{cfg} T={T}", fmt=fmt, tokens=int(T),
                       **{k: v for k, v in m.items() if k != "adjusted"}, adjusted=m.get("adjusted")))


GATE_SHAPES = [
    # (T, d, d_real, f, E, k): one-workgroup routing with split partials, with the
    # router's in-place top-k (one 128-column group), the per-token finisher,
    # and several tiles with the in-place top-k
    (64, 256, 256, 256, 8, 2),
    (1, 128, 128, 128, 2, 1),
    (513, 384, 384, 512, 7, 3),
    (77, 128, 128, 128, 256, 8),
]
GATE_OPTS = [("softmax_topk", False), ("softmax_topk", True), ("topk_softmax", True)]


@pytest.mark.parametrize("routing,gate_bf16", GATE_OPTS, ids=[f"{r}-bf16{int(b)}" for r, b in GATE_OPTS])
@pytest.mark.parametrize("shape", GATE_SHAPES, ids=[f"T{s[0]}-d{s[1]}-E{s[4]}-k{s[5]}" for s in GATE_SHAPES])
def test_gate_options_vs_oracle(shape, routing, gate_bf16):
    """Softmax over all experts before top-k, and bf16 gate weights: the same
    selection and permutation, the oracle's weights, and the output gates."""
    T, d, dr, f, E, k = shape
    layer = gen.custom_layer(d, f, E, k, d_real=dr, layer_id=3000 + d + f + E + k)
    inp = dict(gen.make_inputs(layer, T=T), routing=routing, gate_bf16=gate_bf16)
    _say(f"[gate] shape={shape} routing={routing} bf16={gate_bf16}")
    dbg = run_debug(inp, "auto")
    ref = parity.oracle_ref(inp)
    parity.check_routing(dbg, ref, T, k, gate_bf16=gate_bf16)
    parity.check_combine_stage(dbg)
    g = parity.bf16_to_f64(dbg["out"])
    m = parity.check_end_to_end(g, dbg, ref, inp, dr)
    _say(f"   out {m}")


def test_gate_options_full_size_decode():
    """The decode-shaped layer with both options (routing of every token)."""
    inp = dict(gen.make_inputs("c1"), routing="softmax_topk", gate_bf16=True)
    T, k = inp["T"], inp["k"]
    dbg = run_debug(inp, "auto")
    ref = parity.oracle_ref(inp)
    parity.check_routing(dbg, ref, T, k, gate_bf16=True)
    g = parity.bf16_to_f64(dbg["out"])
    m = parity.check_end_to_end(g, dbg, ref, inp, inp["d_real"])
    _say(f"[gate] c1 out {m}")
    parity.record(dict(cfg="c1", fmt="block128", routing="softmax_topk", gate_bf16=True,
                       tokens=int(T), **{k: v for k, v in m.items() if k != "adjusted"},
                       adjusted=m.get("adjusted")))


@pytest.mark.parametrize("fmt", FMTS)
def test_deterministic_bits(fmt):
    layer = gen.custom_layer(256, 256, 8, 2, layer_id=2000)
    inp = gen.make_inputs(layer, T=700, fmt=fmt)
    p = moe.device_inputs(inp)
    args = (p["x"], p["W_router"], p["b_router"], p["k"], p["W_gateup"], p["S_gateup"],
            p["b_gateup"], p["W_down"], p["S_down"], p["b_down"])
    for path in ("prefill", "decode"):
        a = moe.forward(*args, path=path, fmt=fmt).clone()
        b = moe.forward(*args, path=path, fmt=fmt).clone()
        torch.cuda.synchronize()
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), path


def test_empty_batch_and_stage_split():
    layer = gen.custom_layer(256, 256, 8, 2, layer_id=2001)
    inp = gen.make_inputs(layer, T=40)
    p = moe.device_inputs(inp)
    args = (p["W_router"], p["b_router"], p["k"], p["W_gateup"], p["S_gateup"], p["b_gateup"],
            p["W_down"], p["S_down"], p["b_down"])
    empty = torch.empty((0, 256), dtype=torch.bfloat16, device="cuda")
    assert moe.forward(empty, *args).shape == (0, 256)
    whole = moe.forward(p["x"], *args)
    ws = torch.empty(moe.workspace_bytes(40, 256, 256, 8, 2), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(whole)
    moe.forward_stages("router", "place", p["x"], *args, out, ws)
    moe.forward_stages("gateup", "gateup", p["x"], *args, out, ws)
    moe.forward_stages("down", "combine", p["x"], *args, out, ws)
    torch.cuda.synchronize()
    assert torch.equal(whole.view(torch.int16), out.view(torch.int16))


FULL = [(c, "block128") for c in ["c1", "c2", "c3", "c4a", "c4b"]] + \
       [(c, "mx") for c in ["c1", "c2", "c3", "c4a", "c4b"]] + \
       [(c, "mxfp4") for c in ["c1", "c2", "c3", "c4a", "c4b"]]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("cfg,fmt", FULL, ids=[f"{c}-{f}" for c, f in FULL])
def test_full_size_sampled(cfg, fmt):
    """Full-size workload in the benchmark's launch configuration (auto path):
    routing and x quantisation on every token; the expert math on a seeded
    sample of tokens plus the first and last row of every expert's last row
    tile (the ragged tails of both GEMMs' tile lists)."""
    c = gen.CONFIGS[cfg]
    _say(f"[full] {cfg} {fmt}: generating inputs T={c.T} d={c.layer.d} f={c.layer.f} "
         f"E={c.layer.E} k={c.layer.k}")
    inp = gen.make_inputs(cfg, fmt=fmt)
    T, k, dr = inp["T"], inp["k"], inp["d_real"]
    _say(f"[full] {cfg}: running the HIP path")
    dbg = run_debug(inp, "auto")
    _say(f"[full] {cfg}: oracle routing + x quantisation on all {T} tokens")
    r = parity.orc.route(inp)
    parity.check_routing(dbg, r, T, k)
    x32 = gen.bf16_bits_to_f32(inp["x"])
    xq, xs = parity.orc.FORMATS[fmt][0](x32)
    parity.check_xquant(dbg, xq, xs)
    rng = np.random.default_rng(12345)
    edges = parity.tile_edge_tokens(r["offsets"], r["row_token"])
    sample = np.unique(np.concatenate([[0, T - 1], rng.choice(T, size=min(T, 160), replace=False), edges]))
    _say(f"[full] {cfg}: oracle expert math on {len(sample)} sampled tokens ({len(edges)} at tile edges)")
    ref = parity.oracle_ref(inp, tokens=sample)
    nflip, ncodes = parity.check_h_decisions(dbg, ref, fmt)
    worst = parity.check_down_stage(dbg, ref, inp, dr)
    parity.check_combine_stage(dbg, sample)
    g = parity.bf16_to_f64(dbg["out"])[sample]
    m = parity.check_end_to_end(g, dbg, ref, inp, dr)
    _say(f"[full] {cfg} {fmt}: out {m}\n   h decisions differing from the oracle: {nflip}/{ncodes}; "
         f"down-stage err/bound {worst:.3f}")
    parity.record(dict(cfg=cfg, fmt=fmt, tokens=int(len(sample)), edge_tokens=int(len(edges)),
                       h_flips=int(nflip), h_codes=int(ncodes), down_err_over_bound=worst,
                       **{k: v for k, v in m.items() if k != "adjusted"}, adjusted=m.get("adjusted")))
    assert np.all(g[:, dr:] == 0)


@pytest.mark.timeout(900)
def test_full_size_every_row_c4b():
    """The skewed prefill layer c4b at full size (T=16384, E=128, k=4; the
    hottest expert holds about 14.8 k rows, the tail tiles of the tile lists
    sit behind it) in the benchmark's launch configuration, with the expert
    math checked on every row and token rather than a sample: every GPU h code
    is an admissible rounding of its row's exact h, every down-GEMM row equals
    its definition on the GPU's own h codes, every output token is the combine
    of the GPU's own Y, and the end-to-end gates hold over all tokens."""
    c = gen.CONFIGS["c4b"]
    _say(f"[every-row] c4b: generating inputs T={c.T}")
    inp = gen.make_inputs("c4b", fmt="block128")
    T, k, f, dr = inp["T"], inp["k"], inp["f"], inp["d_real"]
    _say("[every-row] c4b: running the HIP path")
    dbg = run_debug(inp, "auto")
    _say(f"[every-row] c4b: oracle on all {T} tokens")
    ref = parity.oracle_ref(inp)
    parity.check_routing(dbg, ref, T, k)
    parity.check_xquant(dbg, ref["xq"], ref["xs"])
    assert sum(len(it["rows"]) for it in ref["experts"].values()) == T * k
    nflip, ncodes = parity.check_h_decisions(dbg, ref, "block128")
    assert ncodes == T * k * f
    worst = parity.check_down_stage(dbg, ref, inp, dr)
    parity.check_combine_stage(dbg)
    g = parity.bf16_to_f64(dbg["out"])
    m = parity.check_end_to_end(g, dbg, ref, inp, dr)
    _say(f"[every-row] c4b: out {m}\n   h decisions differing from the oracle: {nflip}/{ncodes}; "
         f"down-stage err/bound {worst:.3f}")
    parity.record(dict(cfg="c4b", fmt="block128", tokens=int(T), edge_tokens=0,
                       h_flips=int(nflip), h_codes=int(ncodes), down_err_over_bound=worst,
                       **{k_: v for k_, v in m.items() if k_ != "adjusted"}, adjusted=m.get("adjusted")))
    assert np.all(g[:, dr:] == 0)
