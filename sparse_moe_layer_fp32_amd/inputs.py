"""Seeded synthetic inputs for the sparse MoE block forward.

This module is the one thing the HIP path and the CPU oracle share: it draws
the tensors both sides consume. It holds none of the block's arithmetic
(no routing, no activation quantisation, no expert math, no combine). It does
three input-preparation jobs:

* draws every tensor from its own NumPy ``SeedSequence`` sub-stream, so any
  tensor (and any single expert's weights) is reproducible on its own;
* converts expert weights statically, as the "GPT-OSS on day 0" post's
  serving formats need: FP8 e4m3 with one fp32 scale per 128x128 block
  (section "GPT-OSS on Hopper"), or MXFP8 with one E8M0 power-of-two scale
  per 32 rows of K per column (the "Hosting Qwen on Blackwell" post, section
  "Quantization": microscaling, weights converted statically), both rounded by PyTorch's ``float8_e4m3fn`` cast (a
  library routine), or MXFP4 (section "GPT-OSS on Hopper": the checkpoints
  ship in MXFP4): E2M1 codes with the same scale blocks, rounded here by a
  nearest-value search, packed two per byte along K;
* conditions the router inputs: rows of ``x`` whose k-th and (k+1)-th fp64
  router logits lie within ``MARGIN`` are redrawn, so the top-k set of every
  token is unambiguous at fp32 accuracy; for the skewed-load layer the router
  bias is calibrated so that expert popularity follows a Zipf law.

Distributions (variance notation ``N(0, 1/n)``; ``0.1`` and ``0.02`` are
standard deviations): x ~ N(0,1) -> bf16; W_router ~ N(0, 1/d_real) fp32;
b_router ~ N(0, 0.1^2) fp32; gate/up ~ N(0, 1/d_real); down ~ N(0, 1/f);
expert biases ~ N(0, 0.02^2) -> bf16.  Hidden sizes that are not a multiple
of 128 are padded with zero columns (x, router rows, gate/up rows, down
columns and down bias), so the padded outputs are exactly zero.
"""
from __future__ import annotations

import hashlib
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np
import torch

MARGIN = 1e-3          # fp64 gap required between the k-th and (k+1)-th logit
FP8_MAX = 448.0        # largest finite e4m3 (OCP "fn") magnitude
BLOCK = 128            # weight block edge and activation group width

# sub-stream tags
_T_WR, _T_BR, _T_WGU, _T_WDN, _T_BGU, _T_BDN, _T_X, _T_XRE, _T_PERM, _T_CAL = range(1, 11)


@dataclass(frozen=True)
class Layer:
    """Shape of one MoE layer; ``layer_id`` keys the weight sub-streams."""
    name: str
    layer_id: int
    d: int            # hidden size as stored (multiple of 128)
    d_real: int       # hidden size before zero padding
    f: int            # expert intermediate size (multiple of 128)
    E: int            # number of experts
    k: int            # experts per token
    router: str = "gauss"   # "gauss" or "zipf"
    zipf_s: float = 1.1


@dataclass(frozen=True)
class Config:
    name: str
    layer: Layer
    T: int
    role: str          # "parity", "decode" or "prefill"


_L0 = Layer("tiny", 0, 256, 256, 256, 8, 2)
_L1 = Layer("gpt-oss-20b-like", 1, 2944, 2880, 2944, 32, 4)
_L3 = Layer("qwen3-235b-like", 3, 4096, 4096, 1536, 128, 8)
_L4 = Layer("gpt-oss-120b-like-zipf", 4, 2944, 2880, 2944, 128, 4, router="zipf")

CONFIGS = {
    "c0": Config("c0", _L0, 64, "parity"),
    "c1": Config("c1", _L1, 64, "decode"),
    "c2": Config("c2", _L1, 8192, "prefill"),
    "c3": Config("c3", _L3, 4096, "prefill"),
    "c4a": Config("c4a", _L4, 256, "decode"),
    "c4b": Config("c4b", _L4, 16384, "prefill"),
}


def custom_layer(d, f, E, k, d_real=None, layer_id=100, router="gauss"):
    """A layer of arbitrary shape for small parity cases."""
    return Layer(f"custom-{d}-{f}-{E}-{k}", layer_id, d, d if d_real is None else d_real,
                 f, E, k, router)


def _rng(seed, *tags):
    return np.random.default_rng(np.random.SeedSequence([int(seed)] + [int(t) for t in tags]))


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round-to-nearest-even, via PyTorch."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f32(u: np.ndarray) -> np.ndarray:
    return (u.astype(np.uint32) << 16).view(np.float32)


def quantize_weight_blocks(w: np.ndarray):
    """Static FP8 conversion of one expert matrix ``w`` [K, N] (fp32).

    One fp32 scale per 128x128 block: ``s = amax/448`` (1.0 for an all-zero
    block), codes = e4m3(clamp(w/s, +-448)) with round-to-nearest-even.
    Returns (codes uint8 [K, N], scales fp32 [K/128, N/128]).
    """
    K, N = w.shape
    t = torch.from_numpy(w).view(K // BLOCK, BLOCK, N // BLOCK, BLOCK)
    amax = t.abs().amax(dim=(1, 3))
    s = torch.where(amax > 0, amax / FP8_MAX, torch.ones_like(amax))
    q = (t / s.view(K // BLOCK, 1, N // BLOCK, 1)).clamp_(-FP8_MAX, FP8_MAX)
    codes = q.to(torch.float8_e4m3fn).view(torch.uint8).reshape(K, N).numpy()
    return codes, s.numpy().astype(np.float32)


MX_BLOCK = 32         # MX block length along K


def quantize_weight_mx(w: np.ndarray):
    """Static MXFP8 conversion of one expert matrix ``w`` [K, N] (fp32).

    One E8M0 scale 2^e per 32 consecutive K rows of a column, e the smallest
    exponent with amax <= 448 * 2^e (amax = m * 2^p with m in [0.5, 1):
    e = p - 9 if m <= 0.875, else p - 8), 2^-127 for an all-zero block;
    codes = e4m3(w / 2^e), round-to-nearest-even.
    Returns (codes uint8 [K, N], E8M0 codes uint8 [K/32, N]).
    """
    K, N = w.shape
    t = torch.from_numpy(w).double().view(K // MX_BLOCK, MX_BLOCK, N)
    amax = t.abs().amax(dim=1)
    m, p = torch.frexp(amax)
    e = torch.where(m <= 0.875, p - 9, p - 8)
    e = torch.where(amax > 0, e, torch.full_like(e, -127)).clamp(-127, 127)
    q = t / torch.ldexp(torch.ones_like(amax), e).view(K // MX_BLOCK, 1, N)
    codes = q.float().to(torch.float8_e4m3fn).view(torch.uint8).reshape(K, N).numpy()
    return codes, (e + 127).to(torch.uint8).numpy()


_E2M1_MAGS = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def _e2m1_round(q: np.ndarray) -> np.ndarray:
    """Nearest E2M1 code (ties to the even code), sign in bit 3; |q| <= 6."""
    a = np.abs(q)
    lo = np.clip(np.searchsorted(_E2M1_MAGS, a, side="right") - 1, 0, 7)
    hi = np.minimum(lo + 1, 7)
    dlo, dhi = a - _E2M1_MAGS[lo], _E2M1_MAGS[hi] - a
    up = (dhi < dlo) | ((dhi == dlo) & (lo % 2 == 1))
    idx = np.where(up & (hi != lo), hi, lo).astype(np.uint8)
    return idx | np.where(np.signbit(q), 8, 0).astype(np.uint8)


def quantize_weight_mxfp4(w: np.ndarray):
    """Static MXFP4 conversion of one expert matrix ``w`` [K, N] (fp32).

    One E8M0 scale 2^e per 32 consecutive K rows of a column, e the smallest
    exponent with amax <= 6 * 2^e (amax = m * 2^p with m in [0.5, 1):
    e = p - 3 if m <= 0.75, else p - 2), 2^-127 for an all-zero block; codes =
    E2M1 nearest of w / 2^e, two per byte along K (low nibble = even K).
    Returns (packed uint8 [K/2, N], E8M0 codes uint8 [K/32, N]).
    """
    K, N = w.shape
    t = np.asarray(w, np.float64).reshape(K // MX_BLOCK, MX_BLOCK, N)
    amax = np.abs(t).max(axis=1)
    m, p = np.frexp(amax)
    e = np.where(m <= 0.75, p - 3, p - 2)
    e = np.clip(np.where(amax > 0, e, -127), -127, 127)
    codes = _e2m1_round(t / np.ldexp(1.0, e)[:, None, :]).reshape(K, N)
    packed = (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8)
    return packed, (e + 127).astype(np.uint8)


def _draw_router(layer: Layer, seed: int):
    d, dr, E = layer.d, layer.d_real, layer.E
    Wr = np.zeros((d, E), np.float32)
    Wr[:dr] = _rng(seed, layer.layer_id, _T_WR).standard_normal((dr, E), dtype=np.float32) \
        * np.float32(1.0 / np.sqrt(dr))
    br = (_rng(seed, layer.layer_id, _T_BR).standard_normal(E, dtype=np.float32)
          * np.float32(0.1)).astype(np.float32)
    return Wr, br


def _draw_x_rows(layer: Layer, n: int, rng) -> np.ndarray:
    x = np.zeros((n, layer.d), np.float32)
    x[:, :layer.d_real] = rng.standard_normal((n, layer.d_real), dtype=np.float32)
    return to_bf16_bits(x)


def _kth_gap(logits: np.ndarray, k: int) -> np.ndarray:
    """Per row: (k-th largest) - ((k+1)-th largest); +inf when k == E."""
    E = logits.shape[1]
    if k >= E:
        return np.full(logits.shape[0], np.inf)
    part = -np.partition(-logits, (k - 1, k), axis=1)
    return part[:, k - 1] - part[:, k]


def _router_logits64(xbits, Wr, br):
    return bf16_bits_to_f32(xbits).astype(np.float64) @ Wr.astype(np.float64) + br.astype(np.float64)


def zipf_targets(layer: Layer, seed: int) -> np.ndarray:
    """Target popularity share of every expert: p_r ~ r^-s over a seeded permutation."""
    E = layer.E
    ranks = np.arange(1, E + 1, dtype=np.float64)
    p = ranks ** (-layer.zipf_s)
    p /= p.sum()
    perm = _rng(seed, layer.layer_id, _T_PERM).permutation(E)
    target = np.empty(E)
    target[perm] = p          # expert perm[r] gets rank r+1
    return target


def _calibrate_zipf_bias(layer: Layer, seed: int, Wr: np.ndarray, n_cal=16384, iters=200):
    """Router bias that makes top-k popularity follow ``zipf_targets``.

    Fixed-point iteration on a calibration batch drawn from its own
    sub-stream: b_e += 0.5*(log(n*k*p_e + 0.5) - log(count_e + 0.5)).
    """
    p = zipf_targets(layer, seed)
    xc = _draw_x_rows(layer, n_cal, _rng(seed, layer.layer_id, _T_CAL))
    L0 = bf16_bits_to_f32(xc).astype(np.float64) @ Wr.astype(np.float64)
    b = np.log(p)
    k = layer.k
    for _ in range(iters):
        sel = np.argpartition(-(L0 + b), k - 1, axis=1)[:, :k]
        counts = np.bincount(sel.ravel(), minlength=layer.E)
        b += 0.5 * (np.log(n_cal * k * p + 0.5) - np.log(counts + 0.5))
    b -= b.mean()
    return b.astype(np.float32)


def draw_x(layer: Layer, T: int, seed: int, Wr, br, margin=MARGIN):
    """x [T, d] bf16 bits, with every row meeting the top-k margin rule."""
    x = _draw_x_rows(layer, T, _rng(seed, layer.layer_id, _T_X, T))
    if T == 0:
        return x
    gap = _kth_gap(_router_logits64(x, Wr, br), layer.k)
    redrawn = 0
    for t in np.nonzero(gap <= margin)[0]:
        attempt = 0
        while True:
            row = _draw_x_rows(layer, 1, _rng(seed, layer.layer_id, _T_XRE, T, t, attempt))
            if _kth_gap(_router_logits64(row, Wr, br), layer.k)[0] > margin:
                x[t] = row[0]
                redrawn += 1
                break
            attempt += 1
    return x


def _expert_weights(layer: Layer, seed: int, e: int, fmt: str = "block128"):
    d, dr, f = layer.d, layer.d_real, layer.f
    wgu = np.zeros((d, 2 * f), np.float32)
    wgu[:dr] = _rng(seed, layer.layer_id, _T_WGU, e).standard_normal((dr, 2 * f), dtype=np.float32)
    wgu[:dr] *= np.float32(1.0 / np.sqrt(dr))
    wdn = np.zeros((f, d), np.float32)
    wdn[:, :dr] = _rng(seed, layer.layer_id, _T_WDN, e).standard_normal((f, dr), dtype=np.float32)
    wdn[:, :dr] *= np.float32(1.0 / np.sqrt(f))
    conv = {"mx": quantize_weight_mx, "mxfp4": quantize_weight_mxfp4}.get(fmt, quantize_weight_blocks)
    return conv(wgu), conv(wdn)


_WEIGHT_CACHE: dict = {}


def make_weights(layer: Layer, seed: int = 0, workers: int | None = None, cache: bool = True,
                 fmt: str = "block128"):
    """All layer parameters as NumPy arrays (FP8 codes as uint8, bf16 as uint16 bits).
    ``fmt``: "block128" (fp32 scales per 128x128 block), "mx" (E8M0 scales
    per 32 K rows per column) or "mxfp4" (E2M1 codes packed two per byte
    along K, the same E8M0 scales); the underlying fp32 draws are the same."""
    if fmt not in ("block128", "mx", "mxfp4"):
        raise ValueError(f"unknown weight format {fmt!r}")
    key = (layer, seed, fmt)
    if cache and key in _WEIGHT_CACHE:
        return _WEIGHT_CACHE[key]
    d, f, E = layer.d, layer.f, layer.E
    Wr, br = _draw_router(layer, seed)
    if layer.router == "zipf":
        br = _calibrate_zipf_bias(layer, seed, Wr)
    kp = 2 if fmt == "mxfp4" else 1      # K rows per stored byte row
    Wgu = np.empty((E, d // kp, 2 * f), np.uint8)
    Wdn = np.empty((E, f // kp, d), np.uint8)
    if fmt in ("mx", "mxfp4"):
        Sgu = np.empty((E, d // MX_BLOCK, 2 * f), np.uint8)
        Sdn = np.empty((E, f // MX_BLOCK, d), np.uint8)
    else:
        Sgu = np.empty((E, d // BLOCK, 2 * f // BLOCK), np.float32)
        Sdn = np.empty((E, f // BLOCK, d // BLOCK), np.float32)

    def job(e):
        (Wgu[e], Sgu[e]), (Wdn[e], Sdn[e]) = _expert_weights(layer, seed, e, fmt)

    workers = workers or min(16, len(os.sched_getaffinity(0)))
    if E * d * f > (1 << 22):
        with ThreadPoolExecutor(workers) as ex:
            list(ex.map(job, range(E)))
    else:
        for e in range(E):
            job(e)
    bgu = np.asarray(_rng(seed, layer.layer_id, _T_BGU).standard_normal((E, 2 * f), dtype=np.float32)
                     * np.float32(0.02), np.float32)
    bdn = np.zeros((E, d), np.float32)
    bdn[:, :layer.d_real] = _rng(seed, layer.layer_id, _T_BDN).standard_normal(
        (E, layer.d_real), dtype=np.float32) * np.float32(0.02)
    w = dict(W_router=Wr, b_router=br, W_gateup=Wgu, S_gateup=Sgu, b_gateup=to_bf16_bits(bgu),
             W_down=Wdn, S_down=Sdn, b_down=to_bf16_bits(bdn))
    if cache:
        _WEIGHT_CACHE.clear()
        _WEIGHT_CACHE[key] = w
    return w


def make_inputs(cfg, seed: int = 0, T: int | None = None, margin=MARGIN, fmt: str = "block128"):
    """Full input set for a named config (``"c0"`` ...) or a (Layer, T) pair.

    Returns a dict with the layer shape (T, d, d_real, f, E, k), the weight
    ``format`` and the arrays x (bf16 bits [T,d]), W_router [d,E], b_router [E],
    W_gateup (e4m3 [E,d,2f]), S_gateup, b_gateup (bf16 bits [E,2f]), W_down
    (e4m3 [E,f,d]), S_down, b_down (bf16 bits [E,d]).  Scales: "block128"
    fp32 [E,d/128,2f/128] and [E,f/128,d/128]; "mx" E8M0 uint8 [E,d/32,2f]
    and [E,f/32,d]; "mxfp4" the same scales with W_gateup [E,d/2,2f] and
    W_down [E,f/2,d] holding two E2M1 codes per byte along K.
    """
    if isinstance(cfg, str):
        c = CONFIGS[cfg]
        layer, T = c.layer, (c.T if T is None else T)
    else:
        layer = cfg
        assert T is not None
    w = make_weights(layer, seed, fmt=fmt)
    x = draw_x(layer, T, seed, w["W_router"], w["b_router"], margin)
    out = dict(T=T, d=layer.d, d_real=layer.d_real, f=layer.f, E=layer.E, k=layer.k, x=x, format=fmt)
    out.update(w)
    return out


def digest(inputs: dict) -> dict:
    """SHA-256 of every array in an input set (for reproducibility records)."""
    return {k: hashlib.sha256(np.ascontiguousarray(v).tobytes()).hexdigest()
            for k, v in sorted(inputs.items()) if isinstance(v, np.ndarray)}


# ----------------------------------------------------------------------------- attention with sinks
_T_AQ, _T_AK, _T_AV, _T_ASINK, _T_ALEN = range(20, 25)


@dataclass(frozen=True)
class AttnShape:
    """GQA attention shape: query heads, key/value heads, head dim."""
    name: str
    Hq: int
    Hkv: int
    D: int = 64


GPT_OSS_ATTN = AttnShape("gpt-oss-like", 64, 8, 64)


def attn_sinks(shape: AttnShape, seed: int = 0) -> np.ndarray:
    """Per-head sink logits, fp32 ~ N(0, 1) (learned values of a few units)."""
    return (_rng(seed, _T_ASINK, shape.Hq).standard_normal(shape.Hq, dtype=np.float32)).astype(np.float32)


def make_attn_prefill(shape: AttnShape, S: int, seed: int = 0) -> dict:
    """One sequence: q [S, Hq, D], k and v [S, Hkv, D] (bf16 bits, token major),
    sinks [Hq] fp32, sm_scale = 1/sqrt(D).  q, k ~ N(0, 1), v ~ N(0, 1)."""
    r = lambda t, shp: to_bf16_bits(_rng(seed, t, S, shape.Hq).standard_normal(shp, dtype=np.float32))
    return dict(kind="prefill", S=S, Hq=shape.Hq, Hkv=shape.Hkv, D=shape.D,
                q=r(_T_AQ, (S, shape.Hq, shape.D)), k=r(_T_AK, (S, shape.Hkv, shape.D)),
                v=r(_T_AV, (S, shape.Hkv, shape.D)), sinks=attn_sinks(shape, seed),
                sm_scale=float(1.0 / np.sqrt(shape.D)))


def make_attn_decode(shape: AttnShape, B: int, Lmax: int, seed: int = 0, ragged: bool = True) -> dict:
    """B sequences, one query each: q [B, Hq, D]; caches [B, Hkv, Lmax, D]
    (heads major, tokens contiguous); kv_len [B] in [1, Lmax] (uniform over
    [Lmax/2, Lmax] when ragged, else Lmax)."""
    r = lambda t, shp: to_bf16_bits(_rng(seed, t, B, Lmax).standard_normal(shp, dtype=np.float32))
    if ragged:
        kv_len = _rng(seed, _T_ALEN, B, Lmax).integers(max(1, Lmax // 2), Lmax + 1, size=B).astype(np.int32)
    else:
        kv_len = np.full(B, Lmax, np.int32)
    return dict(kind="decode", B=B, Lmax=Lmax, Hq=shape.Hq, Hkv=shape.Hkv, D=shape.D,
                q=r(_T_AQ, (B, shape.Hq, shape.D)), k=r(_T_AK, (B, shape.Hkv, Lmax, shape.D)),
                v=r(_T_AV, (B, shape.Hkv, Lmax, shape.D)), kv_len=kv_len, sinks=attn_sinks(shape, seed),
                sm_scale=float(1.0 / np.sqrt(shape.D)))
