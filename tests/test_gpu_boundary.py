"""Boundary conventions of the C ABI on the GPU: graph capture and NaN inputs.

* Graph capture: the forward enqueues kernels only (no host sync, no
  allocation, no memset), so a HIP graph captured after one eager warm-up
  call replays it bit for bit, also after new input values are copied into
  the captured buffers ("Fast embeddings on GPUs", section "CUDA graph
  management": an eager warm-up, then capture, then replays; "GPT-OSS on day
  0", opening of section "Kernels for GPT-OSS": the CUDA-graph framework
  serves the new model unchanged).  Every replay is compared with the eager
  result, with eager work and synchronisations between the replays.
* NaN: a NaN in x makes its token's outputs NaN, a NaN in an expert's gate/up
  weights makes the outputs of the tokens routed to it NaN, the expert
  indices stay valid and distinct, and every other token's output keeps the
  bits of the NaN-free run; the NaN pattern of the output equals the
  oracle's.
"""
import sys

import numpy as np
import pytest
import torch

import sparse_moe_layer_fp32_amd as moe
from sparse_moe_layer_fp32_amd import inputs as gen
from tests import parity

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _bits(t):
    return t.view(torch.int16)


def _graph_inputs(case, fmt):
    if case == "schedule":  # prefill tile lists that go through the per-XCD tile counters
        layer = gen.custom_layer(768, 512, 256, 8, layer_id=7000, router="zipf")
        return gen.make_inputs(layer, T=1024, fmt=fmt), "prefill"
    return gen.make_inputs(case, fmt=fmt), "auto"


@pytest.mark.parametrize("cfg", ["c0", "c1", "schedule"])
@pytest.mark.parametrize("fmt", ["block128", "mx"])
def test_graph_capture_replays_bit_equal(cfg, fmt):
    """c0 and c1: one-router-tile batches; "schedule": a prefill batch whose
    GEMM tile counters the place stage zeroes and the last workgroup zeroes
    again in every replay."""
    _say(f"[graph] {cfg} {fmt}")
    inp, path = _graph_inputs(cfg, fmt)
    p = moe.device_inputs(inp)
    blk = moe.MoeBlock(p)
    T, d = inp["T"], inp["d"]
    x = p["x"].clone()
    ws = blk.workspace(T)
    out_eager = torch.empty((T, d), dtype=torch.bfloat16, device="cuda")
    blk(x, out=out_eager, path=path)            # eager warm-up
    torch.cuda.synchronize()
    ref = out_eager.clone()

    out_g = torch.empty_like(out_eager)
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        blk(x, out=out_g, path=path)            # warm-up on the capture stream's side
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        blk(x, out=out_g, path=path)
    assert blk.workspace(T) is ws               # the captured workspace is the one in use

    for rep in range(3):
        out_g.fill_(0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(_bits(out_g), _bits(ref)), f"replay {rep} differs from the eager call"
        out_eager.fill_(0)
        blk(x, out=out_eager, path=path)        # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(_bits(out_eager), _bits(ref))

    # new token values in the captured input buffer: the replay recomputes
    x2 = torch.roll(p["x"], shifts=1, dims=0).contiguous()
    ref2 = blk(x2, out=torch.empty_like(out_eager), path=path).clone()
    torch.cuda.synchronize()
    x.copy_(x2)
    graph.replay()
    torch.cuda.synchronize()
    assert torch.equal(_bits(out_g), _bits(ref2)), "replay on new inputs differs from the eager call"
    assert not torch.equal(_bits(ref2), _bits(ref))


def _check_indices(idx, E):
    assert np.all((idx >= 0) & (idx < E)), "expert index out of range"
    for row in idx:
        assert len(set(row.tolist())) == len(row), f"repeated expert in {row}"


@pytest.mark.parametrize("fmt", ["block128", "mx"])
@pytest.mark.parametrize("path", ["prefill", "decode"])
def test_nan_inputs_propagate(fmt, path):
    layer = gen.custom_layer(256, 256, 8, 2, layer_id=4000)
    T = 40
    base = gen.make_inputs(layer, T=T, fmt=fmt)
    base = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in base.items()}
    E, k = base["E"], base["k"]

    def run(inp):
        p = moe.device_inputs(inp)
        out = moe.forward(p["x"], p["W_router"], p["b_router"], p["k"], p["W_gateup"], p["S_gateup"],
                          p["b_gateup"], p["W_down"], p["S_down"], p["b_down"], path=path, fmt=fmt)
        dbg = moe.forward_debug(p["x"], p["W_router"], p["b_router"], p["k"], p["W_gateup"],
                                p["S_gateup"], p["b_gateup"], p["W_down"], p["S_down"], p["b_down"],
                                path=path, fmt=fmt)
        torch.cuda.synchronize()
        return dbg["topk_idx"].cpu().numpy(), parity.bf16_to_f64(out)

    idx0, out0 = run(base)
    assert np.isfinite(out0).all()
    _check_indices(idx0, E)

    # NaN in one element of x (token 5)
    _say(f"[nan] x element, {fmt} {path}")
    xin = dict(base, x=base["x"].copy())
    xin["x"][5, 17] = 0x7FC0                    # bf16 quiet NaN
    idx, out = run(xin)
    _check_indices(idx, E)
    assert np.isnan(out[5]).all(), "the NaN token's outputs must all be NaN"
    others = np.arange(T) != 5
    np.testing.assert_array_equal(out[others], out0[others])
    np.testing.assert_array_equal(np.sort(idx[others], 1), np.sort(idx0[others], 1))
    ref = parity.oracle_ref(xin)["out64"]
    np.testing.assert_array_equal(np.isnan(out), np.isnan(ref))

    # a NaN weight code in expert 3's gate/up weights
    _say(f"[nan] gate/up weight, {fmt} {path}")
    win = dict(base, W_gateup=base["W_gateup"].copy())
    win["W_gateup"][3, 10, 20] = 0x7F           # e4m3 NaN
    idx, out = run(win)
    _check_indices(idx, E)
    np.testing.assert_array_equal(idx, idx0)
    routed = (idx0 == 3).any(axis=1)
    assert routed.any() and (~routed).any()
    assert np.isnan(out[routed]).all(), "tokens routed to the NaN expert must give NaN"
    np.testing.assert_array_equal(out[~routed], out0[~routed])
    ref = parity.oracle_ref(win)["out64"]
    np.testing.assert_array_equal(np.isnan(out), np.isnan(ref))

    # a NaN router weight: logit 2 is NaN for every token; the picks stay valid and distinct
    _say(f"[nan] router weight, {fmt} {path}")
    rin = dict(base, W_router=base["W_router"].copy())
    rin["W_router"][0, 2] = np.nan
    idx, out = run(rin)
    _check_indices(idx, E)
    picked = (idx == 2).any(axis=1)
    # the NaN logit has one sign for every token: picked by all (positive NaN,
    # above every number) or by none (negative NaN, below every number)
    assert picked.all() or not picked.any(), picked
    assert np.isnan(out[picked]).all()
    # tokens that pick expert 2 in neither run keep their picks and output bits
    keep = ~picked & ~(idx0 == 2).any(axis=1)
    assert keep.any()
    np.testing.assert_array_equal(np.sort(idx[keep], 1), np.sort(idx0[keep], 1))
    np.testing.assert_array_equal(out[keep], out0[keep])
    _say(f"   NaN router logit picked by {'every' if picked.all() else 'no'} token")
