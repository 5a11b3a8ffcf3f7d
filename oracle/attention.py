"""Plain CPU oracle of attention with per-head sinks (test infrastructure only).

Only the test-suite, the package smoke check and the benchmark's CPU-baseline
leg may import this module; it shares no code with the HIP path.

"GPT-OSS on day 0", section "Sink attention": every head carries a learned
sink value that enters the softmax next to the scaled scores, so that
``attn = softmax(q k^T * sm_scale + sink) V``; section "GPT-OSS on Hopper":
the attention is GQA (several query heads share one key/value head).

Readings (also listed in the design notes):
* the sink is one extra logit per head with no value vector: it adds
  ``exp(sink - M)`` to the softmax denominator only;
* prefill attention is causal (query position i sees keys 0..i of its
  sequence); decode has one query per sequence that sees all ``kv_len``
  cached keys (its own already appended);
* query head h reads key/value head ``h // (Hq / Hkv)``;
* ``sm_scale`` is an input (1/sqrt(D) by default in the callers).

Everything is fp64 from the bf16 inputs; the max-subtracted form of the
same section is used, ``M = max(sink, max_j s_j)``.
"""
from __future__ import annotations

import numpy as np

from .codecs import bf16_decode


def sink_softmax_attend(s: np.ndarray, sink: float, v: np.ndarray) -> np.ndarray:
    """One query: scores ``s`` [n] (already scaled and masked to the visible
    keys), the head's sink, values ``v`` [n, D] -> output [D] (fp64)."""
    s = np.asarray(s, np.float64)
    M = max(float(sink), float(s.max())) if s.size else float(sink)
    p = np.exp(s - M)
    denom = np.exp(float(sink) - M) + p.sum()
    return (p @ np.asarray(v, np.float64)) / denom


def prefill(q_bits, k_bits, v_bits, sinks, sm_scale, rows=None):
    """Causal GQA prefill of one sequence.  q [S, Hq, D], k and v [S, Hkv, D]
    as bf16 bits, sinks [Hq] fp32 -> out [len(rows), Hq, D] fp64 for the
    query positions ``rows`` (default: all S)."""
    q, k, v = bf16_decode(q_bits), bf16_decode(k_bits), bf16_decode(v_bits)
    S, Hq, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    rows = np.arange(S) if rows is None else np.asarray(rows)
    out = np.zeros((len(rows), Hq, D))
    for h in range(Hq):
        kh, vh = k[:, h // G], v[:, h // G]
        scores = (q[rows, h] @ kh.T) * float(sm_scale)      # [rows, S]
        for n, i in enumerate(rows):
            out[n, h] = sink_softmax_attend(scores[n, :i + 1], float(sinks[h]), vh[:i + 1])
    return out


def decode(q_bits, k_cache_bits, v_cache_bits, kv_len, sinks, sm_scale):
    """One query per sequence.  q [B, Hq, D]; caches [B, Hkv, Lmax, D] (bf16
    bits, heads major, tokens contiguous); kv_len [B] -> out [B, Hq, D] fp64."""
    q = bf16_decode(q_bits)
    kc, vc = bf16_decode(k_cache_bits), bf16_decode(v_cache_bits)
    B, Hq, D = q.shape
    Hkv = kc.shape[1]
    G = Hq // Hkv
    out = np.zeros((B, Hq, D))
    for b in range(B):
        n = int(kv_len[b])
        for h in range(Hq):
            kh, vh = kc[b, h // G, :n], vc[b, h // G, :n]
            out[b, h] = sink_softmax_attend((kh @ q[b, h]) * float(sm_scale), float(sinks[h]), vh)
    return out
