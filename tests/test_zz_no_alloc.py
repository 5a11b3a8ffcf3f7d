"""moe_forward_noalloc against moe_forward_ex through the C ABI (GPU only).

The allocation-free entry point runs the same kernels on the library's
static device scratch instead of a caller workspace, so on the same inputs
its output must equal the workspace entry point's bit for bit.  Two calls in
a row, the second with a smaller batch (the scratch keeps the first call's
contents, which nothing may depend on); device memory is unchanged across a
call once the scratch is set up; sizes beyond the scratch are refused before
anything is enqueued.
"""
import sys

import pytest
import torch

import sparse_moe_layer_fp32_amd as moe
from sparse_moe_layer_fp32_amd import inputs as gen

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _pair(p, fmt, path="auto"):
    args = (p["x"], p["W_router"], p["b_router"], p["k"], p["W_gateup"], p["S_gateup"],
            p["b_gateup"], p["W_down"], p["S_down"], p["b_down"])
    ref = moe.forward(*args, path=path, fmt=fmt)
    out = torch.full_like(ref, float("nan"))
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    moe.forward_noalloc(*args, out, path=path, fmt=fmt)
    torch.cuda.synchronize()
    free1 = torch.cuda.mem_get_info()[0]
    return ref, out, free0, free1


@pytest.mark.parametrize("fmt", ["block128", "mx", "mxfp4"])
def test_noalloc_matches_the_workspace_entry_point(fmt):
    first, second = ("c4a", None), ("c4a", 40)        # 256 tokens, then 40 of the same layer
    for n, (cfg, T) in enumerate((first, second)):
        _say(f"[noalloc] {fmt} call {n + 1}: {cfg} T={T or gen.CONFIGS[cfg].T}")
        inp = gen.make_inputs(cfg, T=T, fmt=fmt)
        p = moe.device_inputs(inp)
        ref, out, free0, free1 = _pair(p, fmt)
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), f"call {n + 1} differs"
        if n == 1:
            assert free1 == free0, "device memory changed across an allocation-free call"


def test_noalloc_decode_and_prefill_paths():
    layer = gen.custom_layer(256, 256, 8, 2, layer_id=5000)
    for T, path in ((700, "prefill"), (33, "decode")):
        _say(f"[noalloc] path={path} T={T}")
        p = moe.device_inputs(gen.make_inputs(layer, T=T))
        ref, out, _, _ = _pair(p, "block128", path)
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), path


def test_noalloc_prefill_tile_counters():
    """A prefill batch whose GEMM tile lists go through the per-XCD tile
    counters (35 MiB of workspace): the counters sit in the shared array and
    must start every call at zero; two calls in a row, the second smaller."""
    layer = gen.custom_layer(768, 512, 256, 8, layer_id=7000, router="zipf")
    for T in (1024, 600):
        _say(f"[noalloc] tile counters T={T}")
        p = moe.device_inputs(gen.make_inputs(layer, T=T))
        ref, out, _, _ = _pair(p, "block128", "prefill")
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), T


def test_noalloc_refuses_sizes_beyond_the_scratch():
    # the prefill-shaped layer needs far more than 64 MiB of workspace: refused on the host
    T, d, f, E, k = 8192, 2944, 2944, 32, 4
    assert moe.workspace_bytes(T, d, f, E, k) > moe.SCRATCH_BYTES
    dev = "cuda"
    x = torch.zeros((T, d), dtype=torch.bfloat16, device=dev)
    Wr = torch.zeros((d, E), dtype=torch.float32, device=dev)
    br = torch.zeros(E, dtype=torch.float32, device=dev)
    Wgu = torch.zeros((E, d, 2 * f), dtype=torch.uint8, device=dev)
    Sgu = torch.ones((E, d // 128, 2 * f // 128), dtype=torch.float32, device=dev)
    bgu = torch.zeros((E, 2 * f), dtype=torch.bfloat16, device=dev)
    Wdn = torch.zeros((E, f, d), dtype=torch.uint8, device=dev)
    Sdn = torch.ones((E, f // 128, d // 128), dtype=torch.float32, device=dev)
    bdn = torch.zeros((E, d), dtype=torch.bfloat16, device=dev)
    out = torch.zeros((T, d), dtype=torch.bfloat16, device=dev)
    with pytest.raises(moe.MoeError) as ei:
        moe.forward_noalloc(x, Wr, br, k, Wgu, Sgu, bgu, Wdn, Sdn, bdn, out)
    assert ei.value.status == -8
    torch.cuda.synchronize()
    assert torch.count_nonzero(out.view(torch.int16)) == 0       # nothing was written
