"""Comparison of the HIP path with the CPU oracle (test infrastructure).

Gates (written here, used by every GPU parity test):
* routing: the top-k expert SET of every token, the expert offsets, the
  permuted row order and the row of every (token, expert) pair are
  bit-identical; gate weights agree per expert to rtol 1e-5 + atol 1e-6
  (fp32 logits on the GPU vs fp64 in the oracle);
* activation quantisation: x codes and scales (fp32 per 128 columns, or E8M0
  per 32 columns for the MXFP8 format) are bit-identical;
* output: with o the oracle's unrounded fp64 output and g the GPU's bf16,
  over the real (unpadded) columns, the mean gate
      sum|g - o| / sum|o| <= 5e-3
  always holds, and the max gate holds in one of three forms, reported by
  name (``check_end_to_end``):
  - "literal":  max|g - o| <= 2e-2 * RMS(o);
  - "bf16-floor": only where the bf16 rounding of o ALONE exceeds the bound
    (max|bf16(o) - o| > 2e-2 * RMS(o): 2e-2 is 5.12 bf16 half-spacings of RMS,
    so rare large outputs near a rounding midpoint cannot meet it in bf16),
    the bound applies to max(|g - o| - |bf16(o) - o|), the error beyond the
    output format's own rounding;
  - "decision-adjusted": the max gate (literal, or bf16-floor under the same
    precondition) against the oracle with its h decisions replaced by the
    GPU's validated ones (``decision_adjusted_reference``): an h code or
    scale is a floating-point-decided integer, taken here in the kernel's
    precision.
  A result that passes only in the third form is a miss of the literal gate,
  and is reported as one.
"""
from __future__ import annotations

import numpy as np

from oracle import codecs
from oracle import oracle as orc

MAX_REL_RMS = 2e-2
MEAN_REL = 5e-3


def bf16_to_f64(t):
    """torch bf16 tensor -> fp64 numpy."""
    import torch
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16).astype(np.uint32).__lshift__(16) \
        .view(np.float32).astype(np.float64)


def output_metrics(g: np.ndarray, o: np.ndarray) -> dict:
    err = np.abs(g - o)
    rms = float(np.sqrt(np.mean(o * o))) if o.size else 0.0
    floor = np.abs(codecs.bf16_round(o) - o)
    return dict(rms=rms, max_err=float(err.max(initial=0.0)),
                max_rel_rms=float(err.max(initial=0.0) / rms) if rms else 0.0,
                max_excess_rel_rms=float(np.max(err - floor, initial=0.0) / rms) if rms else 0.0,
                floor_rel_rms=float(floor.max(initial=0.0) / rms) if rms else 0.0,
                mean_rel=float(err.sum() / np.abs(o).sum()) if o.size and np.abs(o).sum() else 0.0,
                mean_elem_rel=float(np.mean(err / np.maximum(np.abs(o), 1e-30))) if o.size else 0.0)


def check_routing(dbg: dict, ref: dict, T: int, k: int, gate_bf16: bool = False):
    """With ``gate_bf16`` the weights must be bf16 values within one bf16
    spacing (2^-7 relative) of the oracle's: fp32 and fp64 weights that sit
    within ~1e-7 of a rounding midpoint may round to either neighbour; at
    least 99% must be the oracle's exact bf16 value."""
    gi = dbg["topk_idx"].cpu().numpy()
    gw = dbg["topk_w"].cpu().numpy()
    ri, rw = ref["idx"], ref["w"]
    assert gi.shape == (T, k)
    np.testing.assert_array_equal(np.sort(gi, 1), np.sort(ri, 1), err_msg="top-k sets")
    # weights matched by expert
    og = np.argsort(gi, 1)
    orr = np.argsort(ri, 1)
    gws, rws = np.take_along_axis(gw, og, 1), np.take_along_axis(rw, orr, 1)
    if gate_bf16:
        g64 = gws.astype(np.float64)
        np.testing.assert_array_equal(codecs.bf16_round(g64), g64, err_msg="gate weights are bf16")
        np.testing.assert_allclose(g64, rws, rtol=2.0 ** -7, atol=0, err_msg="bf16 gate weights")
        assert np.mean(g64 == rws) >= 0.99, np.mean(g64 == rws)
    else:
        np.testing.assert_allclose(gws, rws, rtol=1e-5, atol=1e-6, err_msg="gate weights")
    np.testing.assert_array_equal(dbg["offsets"].cpu().numpy(), ref["offsets"], err_msg="offsets")
    np.testing.assert_array_equal(dbg["row_token"].cpu().numpy(), ref["row_token"], err_msg="row order")
    # row of each (token, expert)
    grow = dbg["row_of"].cpu().numpy()
    np.testing.assert_array_equal(np.take_along_axis(grow, og, 1), np.take_along_axis(ref["row_of"], orr, 1),
                                  err_msg="row of (token, expert)")


def check_xquant(dbg: dict, ref_xq: np.ndarray, ref_xs: np.ndarray, tokens=None):
    xq = dbg["xq"].cpu().numpy()
    xs = dbg["xs"].cpu().numpy()
    if tokens is not None:
        xq, xs = xq[tokens], xs[tokens]
    np.testing.assert_array_equal(xs, ref_xs, err_msg="x scales")
    bad = np.nonzero(xq != ref_xq)
    assert bad[0].size == 0, (f"x codes differ at {bad[0].size} places, first {list(zip(*bad))[:5]}: "
                              f"gpu {xq[bad][:5]} oracle {ref_xq[bad][:5]}")


def _e4m3_spacing(q):
    """Distance from |q| to the next e4m3 code (in code units)."""
    a = np.maximum(np.abs(q), 2.0 ** -6)
    return np.exp2(np.floor(np.log2(a)) - 3)


# The gfx950 FP8 MFMA multiplies e4m3 pairs exactly but adds the products after
# aligning them to the largest one and truncating ~13 bits below it (measured on
# the device: 32 + 2^-9 gives 32).  The kernel's h therefore differs from the
# exact h by up to a few 1e-4 of the row maximum: up to ~0.2 code units (codes
# span +-448).  An h code is a floating-point decision with several correct
# answers at that precision; a GPU code is admissible when it is a rounding of a
# value within H_CODE_SLACK code units of the exact h.
H_CODE_SLACK = 0.5


# The scales are decisions too: an fp32 scale agrees with the oracle's to
# H_SCALE_RTOL; an E8M0 code must be the MX code of an amax within H_SCALE_RTOL
# of the exact block amax.  For MX the code slack is kept in absolute terms,
# H_CODE_SLACK units of the 128-column group's amax/448, since the GEMM's
# accumulation error does not depend on how h is quantised afterwards.
H_SCALE_RTOL = 5e-4


def _fmt(inp_or_ref) -> str:
    return inp_or_ref.get("format", "block128")


def check_h_decisions(dbg: dict, ref: dict, fmt: str = "block128"):
    """Every GPU h code is an admissible rounding of the oracle's exact h; the
    scales agree to the accumulation error.  Returns the number of codes that
    differ from the oracle's own decisions (reported, not gated)."""
    hq = dbg["hq"].cpu().numpy()
    hs = dbg["hs"].cpu().numpy()
    n_diff = n = 0
    for e, it in ref["experts"].items():
        rows = it["rows"]
        h = it["h"]
        qg = codecs.e4m3_decode(hq[rows])
        if fmt in ("mx", "mxfp4"):
            amax = np.abs(h).reshape(len(rows), -1, 32).max(axis=2)
            lo = orc.mx_scale_exponent(amax * (1 - H_SCALE_RTOL)) + 127
            hi = orc.mx_scale_exponent(amax * (1 + H_SCALE_RTOL)) + 127
            c = hs[rows].astype(np.int64)
            assert np.all((c >= lo) & (c <= hi)), f"h E8M0 scales expert {e}"
            sg = np.repeat(codecs.e8m0_decode(hs[rows]), 32, axis=1)
            unit = np.repeat(np.abs(h).reshape(len(rows), -1, 128).max(axis=2) / 448.0, 128, axis=1)
        else:
            np.testing.assert_allclose(hs[rows], it["hs"], rtol=H_SCALE_RTOL,
                                       err_msg=f"h scales expert {e}")
            sg = unit = np.repeat(hs[rows].astype(np.float64), 128, axis=1)
        # |GPU value - exact h| within one code spacing plus the slack
        bad = np.abs(qg * sg - h) > _e4m3_spacing(qg) * sg + H_CODE_SLACK * unit
        assert not bad.any(), (f"h codes expert {e}: gpu {qg[bad][:8]} exact {(h / sg)[bad][:8]}")
        n_diff += int((hq[rows] != it["hq"]).sum())
        n += hq[rows].size
    return n_diff, n


def check_down_stage(dbg: dict, ref: dict, inp: dict, d_real: int):
    """The down GEMM output of every evaluated row equals its definition applied
    to the GPU's own (validated) h codes: deq(hq, hs) @ deq(W_down) + b_down,
    within the FP8 MFMA accumulation error (2^-10 of the sum of |terms|)."""
    _, deq, wdeq = orc.FORMATS[_fmt(inp)]
    hq = dbg["hq"].cpu().numpy()
    hs = dbg["hs"].cpu().numpy()
    y = dbg["y"].cpu().numpy()
    worst = 0.0
    for e, it in ref["experts"].items():
        rows = it["rows"]
        hdeq = deq(hq[rows], hs[rows])
        W = wdeq(inp["W_down"][e], inp["S_down"][e])
        want = hdeq @ W + codecs.bf16_decode(inp["b_down"][e])
        bound = 2.0 ** -10 * (np.abs(hdeq) @ np.abs(W)) + 1e-6
        err = np.abs(y[rows] - want)
        worst = max(worst, float((err / bound).max()))
        assert np.all(err <= bound), f"down GEMM expert {e}: max err/bound {(err / bound).max():.3f}"
        assert np.all(y[rows][:, d_real:] == 0)
    return worst


def check_combine_stage(dbg: dict, tokens=None):
    """out = bf16(sum_j w_j Y[row_of(t, j)]) from the GPU's own w and Y: the
    fp32 sum rounded once to bf16 (within one bf16 spacing)."""
    w = dbg["topk_w"].cpu().numpy().astype(np.float64)
    rows = dbg["row_of"].cpu().numpy()
    y = dbg["y"].cpu().numpy().astype(np.float64)
    out = bf16_to_f64(dbg["out"])
    tok = np.arange(out.shape[0]) if tokens is None else np.asarray(tokens)
    want = np.einsum("tk,tkd->td", w[tok], y[rows[tok]])
    mag = np.einsum("tk,tkd->td", np.abs(w[tok]), np.abs(y[rows[tok]]))   # fp32 sum error scale
    spacing = np.exp2(np.floor(np.log2(np.maximum(np.abs(want), 1e-30))) - 7)
    err = np.abs(out[tok] - want)
    assert np.all(err <= spacing + 1e-6 * mag), f"combine: worst {np.max(err - spacing - 1e-6 * mag)}"


def decision_adjusted_reference(dbg: dict, ref: dict, inp: dict):
    """The oracle's output with its h decisions replaced by the GPU's validated
    ones (the only freedom the method leaves): out + sum_j w_j (deq(hq_gpu) -
    deq(hq_oracle)) @ deq(W_down), per evaluated token."""
    _, deq, wdeq = orc.FORMATS[_fmt(inp)]
    hq = dbg["hq"].cpu().numpy()
    hs = dbg["hs"].cpu().numpy()
    tok = ref["tokens"]
    pos_of = {int(t): i for i, t in enumerate(tok)}
    adj = ref["out64"].copy()
    row_token = ref["row_token"]
    for e, it in ref["experts"].items():
        rows = it["rows"]
        delta = deq(hq[rows], hs[rows]) - deq(it["hq"], it["hs"])
        if not delta.any():
            continue
        W = wdeq(inp["W_down"][e], inp["S_down"][e])
        dY = delta @ W
        for i, r in enumerate(rows):
            t = int(row_token[r])
            j = int(np.nonzero(ref["row_of"][t] == r)[0][0])
            adj[pos_of[t]] += ref["w"][t, j] * dY[i]
    return adj


def _max_gate(g: np.ndarray, o: np.ndarray, rms: float):
    """(form, max_rel_rms, floor_rel_rms, excess_rel_rms) of the max gate of g
    against o: "literal", "bf16-floor" (only when the floor alone exceeds the
    bound) or None when neither holds."""
    err = np.abs(g - o)
    floor = np.abs(codecs.bf16_round(o) - o)
    mx = float(err.max(initial=0.0) / rms) if rms else 0.0
    fl = float(floor.max(initial=0.0) / rms) if rms else 0.0
    ex = float(np.max(err - floor, initial=0.0) / rms) if rms else 0.0
    if mx <= MAX_REL_RMS:
        return "literal", mx, fl, ex
    if fl > MAX_REL_RMS and ex <= MAX_REL_RMS:
        return "bf16-floor", mx, fl, ex
    return None, mx, fl, ex


def check_end_to_end(g: np.ndarray, dbg: dict, ref: dict, inp: dict, d_real: int) -> dict:
    """The end-to-end accuracy gates against the oracle (module docstring).
    Returns the metrics with ``gate`` = the form of the max gate that holds
    ("literal", "bf16-floor" or "decision-adjusted"); with the last one the
    adjusted metrics are under ``adjusted``."""
    o = ref["out64"][:, :d_real]
    g = g[:, :d_real]
    m = output_metrics(g, o)
    assert m["mean_rel"] <= MEAN_REL, f"out: mean relative error {m}"
    form, *_ = _max_gate(g, o, m["rms"])
    if form is not None:
        m["gate"] = form
        return m
    adj = decision_adjusted_reference(dbg, ref, inp)[:, :d_real]
    aform, amx, afl, aex = _max_gate(g, adj, m["rms"])
    ma = dict(max_rel_rms=amx, floor_rel_rms=afl, max_excess_rel_rms=aex, form=aform,
              mean_rel=float(np.abs(g - adj).sum() / np.abs(o).sum()))
    assert aform is not None, f"out: max error {m}; against the GPU's h decisions {ma}"
    m["gate"] = "decision-adjusted"
    m["adjusted"] = ma
    return m


def record(row: dict):
    """Append one result row (JSON) to the file named by $MOE_PARITY_LOG, if set:
    the full-size parity table is assembled from these rows."""
    import json
    import os
    path = os.environ.get("MOE_PARITY_LOG")
    if path:
        with open(path, "a") as fh:
            fh.write(json.dumps(row) + "\n")


def tile_edge_tokens(offsets: np.ndarray, row_token: np.ndarray, tile_rows=(32, 192)) -> np.ndarray:
    """Tokens of the first and last row of every expert's last row tile, for
    the GEMMs' row-tile heights: the ragged tails of the tile lists."""
    toks = []
    for e in range(len(offsets) - 1):
        c = int(offsets[e + 1] - offsets[e])
        if c == 0:
            continue
        for bm in tile_rows:
            first = int(offsets[e]) + ((c - 1) // bm) * bm
            toks += [int(row_token[first]), int(row_token[int(offsets[e + 1]) - 1])]
    return np.unique(np.asarray(toks, np.int64))


def oracle_ref(inp: dict, tokens=None, keep=True):
    return orc.forward(inp, tokens=tokens, keep=keep)
