"""Formats the rows the full-size GPU parity tests record ($MOE_PARITY_LOG,
one JSON object per line) as the markdown table kept under profiles/.

    MOE_PARITY_LOG=gpurun_out/parity_full_size.jsonl python -m pytest tests -m gpu -k full_size
    python tests/parity_table.py gpurun_out/parity_full_size.jsonl "<command>" > profiles/parity_full_size.md
"""
import json
import sys

HEAD = """# Full-size parity: HIP path vs the CPU oracle, per config and weight format

Command: `{cmd}`

Routing (expert sets, offsets, row order, row of every (token, slot)) and the x
codes and scales are compared on every token and are bit-identical on every
row below.  The expert math is compared on `tokens` sampled tokens: 160 seeded
random ones, the first and last token, and the tokens of the first and last
row of every expert's last row tile for 32- and 192-row tiles (the ragged
tails of both GEMMs' tile lists).  A row whose token count is the config's T
checks the expert math on every row and token.

Columns, with o the oracle's unrounded fp64 output and g the GPU's bf16 output
over the real columns of the sampled tokens:

* `max/RMS` = max|g - o| / RMS(o): the literal max gate is <= 0.02;
* `floor/RMS` = max|bf16(o) - o| / RMS(o), the rounding of o to bf16 alone;
* `excess/RMS` = max(|g - o| - |bf16(o) - o|) / RMS(o);
* `mean rel` = sum|g - o| / sum|o| (gate <= 5e-3, holds on every row);
* `h flips` = h codes that differ from the oracle's own rounding (each GPU
  code is checked to be a rounding of a value within 0.5 code units of the
  exact h);
* `adj max/RMS` = the max error against the oracle with its h decisions
  replaced by the GPU's validated ones (the decision-adjusted reference);
* `gate` = the form of the max gate that holds: literal, bf16-floor (only
  where floor/RMS alone exceeds 0.02) or decision-adjusted.  A row whose gate
  is not "literal" is a MISS of the literal gate.

| config | format | tokens | max/RMS | floor/RMS | excess/RMS | mean rel | h flips | adj max/RMS | gate | literal |
|---|---|---|---|---|---|---|---|---|---|---|
"""


def main(path, cmd):
    rows = [json.loads(line) for line in open(path) if line.strip()]
    out = [HEAD.format(cmd=cmd).rstrip("\n")]
    for r in rows:
        a = r.get("adjusted") or {}
        adj = f"{a['max_rel_rms']:.4f}" if "max_rel_rms" in a else "-"
        flips = f"{r['h_flips']}/{r['h_codes']}" if "h_flips" in r else "-"
        opts = ""
        if r.get("routing") or r.get("gate_bf16"):
            opts = f" ({r.get('routing', '')}{', bf16 w' if r.get('gate_bf16') else ''})"
        out.append(f"| {r['cfg']}{opts} | {r['fmt']} | {r['tokens']} | {r['max_rel_rms']:.4f} | "
                   f"{r['floor_rel_rms']:.4f} | {r['max_excess_rel_rms']:.4f} | {r['mean_rel']:.2e} | "
                   f"{flips} | {adj} | {r['gate']} | {'holds' if r['gate'] == 'literal' else 'MISS'} |")
    print("\n".join(out))


if __name__ == "__main__":
    main(sys.argv[1], sys.argv[2] if len(sys.argv) > 2 else "python -m pytest tests -m gpu")
