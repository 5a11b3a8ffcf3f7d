"""The oracle's pins catch plausible mistakes (CPU only).

Each case plants one mistake into the oracle (monkeypatched for the duration
of the case only) and runs every pin of ``tests/test_oracle_pins.py`` with
all its parameter sets.  At least one pin must fail for every mistake: a
pin set that a dropped bias, a swapped gate/up half, transposed block
scales, a softmax over the wrong set, an unstable permutation, a wrong FP8
maximum, an unquantised h or a wrong sign in silu could all pass would not
pin the oracle.
"""
import inspect
import itertools

import numpy as np
import pytest

from oracle import codecs
from oracle import oracle as orc
from tests import test_oracle_pins as pins


def _pin_calls():
    """(name, function, kwargs) for every pin and every parameter set."""
    calls = []
    for name, fn in inspect.getmembers(pins, inspect.isfunction):
        if not name.startswith("test_") or fn.__module__ != pins.__name__:
            continue
        marks = [m for m in getattr(fn, "pytestmark", []) if m.name == "parametrize"]
        grids = []
        for m in marks:
            names = [n.strip() for n in m.args[0].split(",")] if isinstance(m.args[0], str) else list(m.args[0])
            vals = [v if isinstance(v, (tuple, list)) and len(names) > 1 else (v,) for v in m.args[1]]
            grids.append([dict(zip(names, v)) for v in vals])
        for combo in itertools.product(*grids) if grids else [()]:
            kw = {}
            for d in combo:
                kw.update(d)
            calls.append((name, fn, kw))
    return calls


PIN_CALLS = _pin_calls()


def _failing_pins():
    failed = []
    for name, fn, kw in PIN_CALLS:
        try:
            with np.errstate(all="ignore"):
                fn(**kw)
        except Exception:  # an assertion, or a shape error the mistake causes
            failed.append(f"{name}{kw if kw else ''}")
    return failed


# ------------------------------------------------------------------ planted mistakes
def _drop_gateup_bias(mp):
    orig = orc.expert_mlp

    def bad(xdeq, Wgu_e, Sgu_e, bgu_e, *a, **kw):
        return orig(xdeq, Wgu_e, Sgu_e, np.zeros_like(bgu_e), *a, **kw)
    mp.setattr(orc, "expert_mlp", bad)


def _drop_down_bias(mp):
    orig = orc.expert_mlp

    def bad(xdeq, Wgu_e, Sgu_e, bgu_e, Wdn_e, Sdn_e, bdn_e, *a, **kw):
        return orig(xdeq, Wgu_e, Sgu_e, bgu_e, Wdn_e, Sdn_e, np.zeros_like(bdn_e), *a, **kw)
    mp.setattr(orc, "expert_mlp", bad)


def _drop_router_bias(mp):
    orig = orc.router_logits
    mp.setattr(orc, "router_logits", lambda x, W, b: orig(x, W, np.zeros_like(b)))


def _swap_gate_up(mp):
    """The up half taken as the gate and the gate half as the up projection."""
    def silu_swapped(xdeq, Wgu_e, Sgu_e, bgu_e, Wdn_e, Sdn_e, bdn_e, return_h=False, fmt="block128"):
        quant, deq, wdeq = orc.FORMATS[fmt]
        f = Wgu_e.shape[1] // 2
        P = xdeq @ wdeq(Wgu_e, Sgu_e) + codecs.bf16_decode(bgu_e)
        h = orc.silu(P[:, f:]) * P[:, :f]
        hq, hs = quant(h.astype(np.float32))
        Y = deq(hq, hs) @ wdeq(Wdn_e, Sdn_e) + codecs.bf16_decode(bdn_e)
        return (Y, P, h, hq, hs) if return_h else Y
    mp.setattr(orc, "expert_mlp", silu_swapped)


def _transpose_block_scales(mp):
    def bad(codes, scales):
        K, N = codes.shape
        blk = np.asarray(scales, np.float64).T
        return (codecs.e4m3_decode(codes).reshape(K // orc.GROUP, orc.GROUP, N // orc.GROUP, orc.GROUP)
                * blk[:, None, :, None]).reshape(K, N)
    mp.setattr(orc, "dequant_weight", bad)
    mp.setitem(orc.FORMATS, "block128", (orc.quantize_groups, orc.dequant_groups, bad))


def _softmax_over_all(mp):
    mp.setattr(orc, "gate_weights", orc.gate_weights_all)


def _unstable_permutation(mp):
    """Rows of an expert in descending token order."""
    def bad(idx, E):
        T, k = idx.shape
        flat = idx.reshape(-1).astype(np.int64)
        counts = np.bincount(flat, minlength=E).astype(np.int32)
        offsets = np.zeros(E + 1, np.int32)
        offsets[1:] = np.cumsum(counts)
        order = np.lexsort((-np.arange(T * k), flat))
        row_of = np.empty(T * k, np.int32)
        row_of[order] = np.arange(T * k, dtype=np.int32)
        return counts, offsets, row_of.reshape(T, k), (order // k).astype(np.int32)
    mp.setattr(orc, "permutation", bad)


def _fnuz_maximum(mp):
    mp.setattr(orc, "FP8_MAX", np.float32(240.0))


def _unquantised_h(mp):
    def bad(xdeq, Wgu_e, Sgu_e, bgu_e, Wdn_e, Sdn_e, bdn_e, return_h=False, fmt="block128"):
        quant, deq, wdeq = orc.FORMATS[fmt]
        f = Wgu_e.shape[1] // 2
        P = xdeq @ wdeq(Wgu_e, Sgu_e) + codecs.bf16_decode(bgu_e)
        h = orc.silu(P[:, :f]) * P[:, f:]
        hq, hs = quant(h.astype(np.float32))
        Y = h @ wdeq(Wdn_e, Sdn_e) + codecs.bf16_decode(bdn_e)
        return (Y, P, h, hq, hs) if return_h else Y
    mp.setattr(orc, "expert_mlp", bad)


def _silu_sign(mp):
    mp.setattr(orc, "silu", lambda z: z / (1.0 + np.exp(z)))


def _x_unscaled(mp):
    """Activation codes dequantised without their group scale."""
    mp.setattr(orc, "dequant_groups", lambda c, s: codecs.e4m3_decode(c))
    mp.setitem(orc.FORMATS, "block128", (orc.quantize_groups, orc.dequant_groups, orc.dequant_weight))


MISTAKES = {
    "dropped gate/up bias": _drop_gateup_bias,
    "dropped down bias": _drop_down_bias,
    "dropped router bias": _drop_router_bias,
    "swapped gate/up halves": _swap_gate_up,
    "transposed weight-block scales": _transpose_block_scales,
    "softmax over all experts": _softmax_over_all,
    "unstable permutation": _unstable_permutation,
    "FNUZ maximum 240 instead of 448": _fnuz_maximum,
    "unquantised h": _unquantised_h,
    "wrong sign in silu": _silu_sign,
    "activation scale dropped": _x_unscaled,
}


def test_pins_pass_on_the_unmodified_oracle():
    assert PIN_CALLS and not _failing_pins()


@pytest.mark.parametrize("mistake", sorted(MISTAKES))
def test_planted_mistake_fails_a_pin(mistake, monkeypatch):
    MISTAKES[mistake](monkeypatch)
    failed = _failing_pins()
    assert failed, f"no pin catches: {mistake}"
    print(f"{mistake}: caught by {len(failed)} pin(s), e.g. {failed[:3]}")
