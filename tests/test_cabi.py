"""The C-ABI library loads, exports what include/moe.h declares, and rejects bad
arguments on the host before touching the GPU (CPU only: no compute calls)."""
import ctypes
import os
import re

import pytest

import sparse_moe_layer_fp32_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in ("moe.h", "attention.h")]

OK, ERR_NULL, ERR_SHAPE, ERR_UNSUP, ERR_WS, ERR_ALIGN, ERR_HIP, ERR_FLAGS, ERR_SCRATCH = \
    0, -1, -2, -3, -4, -5, -6, -7, -8


def declared_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*((?:moe|attn)_\w+)\s*\(", text, flags=re.M))
    return sorted(names)


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert set(names) == set(moe.SYMBOLS), names
    L = moe.lib()
    for n in names:
        assert hasattr(L, n), n


def test_status_strings():
    for s in (OK, ERR_NULL, ERR_SHAPE, ERR_UNSUP, ERR_WS, ERR_ALIGN, ERR_HIP, ERR_FLAGS, ERR_SCRATCH):
        assert moe.status_string(s) and moe.status_string(s) != "unknown status"
    assert moe.status_string(-99) == "unknown status"


def test_workspace_bytes():
    assert moe.workspace_bytes(64, 256, 256, 8, 2) > 64 * 256 * (1 + 2 * 4)
    assert moe.workspace_bytes(64, 200, 256, 8, 2) == 0        # d not a multiple of 128
    assert moe.workspace_bytes(64, 256, 256, 8, 9) == 0        # k > 8
    assert moe.workspace_bytes(64, 256, 256, 300, 2) == 0      # E > 256
    assert moe.workspace_bytes(0, 256, 256, 8, 2) > 0
    a = moe.workspace_bytes(100, 256, 384, 8, 2)
    b = moe.workspace_bytes(200, 256, 384, 8, 2)
    assert b > a


# fake, 16-byte aligned device addresses: every case below fails validation
# before any pointer is used, so nothing is dereferenced or launched
FAKE = 1 << 20


def call(T=64, d=256, f=256, E=8, k=2, ws=None, flags=0, null=None, misalign=None, stages=None,
         entry="ex"):
    ptrs = [FAKE + 4096 * i for i in range(11)]
    if null is not None:
        ptrs[null] = None
    if misalign is not None:
        ptrs[misalign] += 4
    if ws is None:
        ws = moe.workspace_bytes(T, d, f, E, k)
    x, Wr, br, Wgu, Sgu, bgu, Wdn, Sdn, bdn, out, wsp = [ctypes.c_void_p(p) if p else None for p in ptrs]
    args = [x, Wr, br, k, Wgu, Sgu, bgu, Wdn, Sdn, bdn, out, T, d, f, E, wsp, ws]
    if stages is not None:
        return moe.lib().moe_forward_stages(*args, flags, stages[0], stages[1], None)
    if entry == "mx":
        return moe.lib().moe_forward_mx(*args, flags, None)
    return moe.lib().moe_forward_ex(*args, flags, None)


@pytest.mark.parametrize("kw,want", [
    (dict(d=200), ERR_SHAPE), (dict(f=100), ERR_SHAPE), (dict(T=-1), ERR_SHAPE), (dict(E=0), ERR_SHAPE),
    (dict(d=0), ERR_SHAPE), (dict(k=0), ERR_UNSUP), (dict(k=9, E=16), ERR_UNSUP),
    (dict(k=5, E=4), ERR_UNSUP), (dict(E=257), ERR_UNSUP), (dict(T=1 << 27, k=4), ERR_UNSUP),
    (dict(d=8320), ERR_UNSUP), (dict(f=8320), ERR_UNSUP), (dict(T=1 << 20, d=4096, k=1), ERR_UNSUP),
    (dict(flags=3), ERR_FLAGS), (dict(flags=32), ERR_FLAGS), (dict(flags=64), ERR_FLAGS), (dict(flags=3 | 4), ERR_FLAGS),
    (dict(flags=1 << 31), ERR_FLAGS), (dict(ws=100), ERR_WS), (dict(null=0), ERR_NULL),
    (dict(null=9), ERR_NULL), (dict(null=10), ERR_NULL), (dict(misalign=3), ERR_ALIGN),
    (dict(misalign=0), ERR_ALIGN), (dict(stages=(3, 2)), ERR_FLAGS), (dict(stages=(0, 6)), ERR_FLAGS),
    (dict(stages=(-1, 2)), ERR_FLAGS),
])
def test_argument_errors(kw, want):
    assert call(**kw) == want


def test_expert_output_buffer_bound():
    # Y (fp32 [T*k, d]) is addressed with 32-bit offsets: 4*T*k*d must stay below
    # 2^31.  d=4096, k=8: T=16383 fits (4*16383*8*4096 < 2^31), T=16384 does not,
    # while every other buffer of these sizes is far below the bound.
    assert moe.workspace_bytes(16383, 4096, 1536, 128, 8) > 0
    assert moe.workspace_bytes(16384, 4096, 1536, 128, 8) == 0
    assert moe.workspace_bytes(16448, 4096, 1536, 128, 8) == 0
    assert call(T=16384, d=4096, f=1536, E=128, k=8, ws=1 << 40) == ERR_UNSUP
    assert call(T=16448, d=4096, f=1536, E=128, k=8, ws=1 << 40, entry="mx") == ERR_UNSUP
    # the skewed gpt-oss-120b-like layer (d=2944, k=4) reaches the bound at T=45591
    assert moe.workspace_bytes(45590, 2944, 2944, 128, 4) > 0
    assert moe.workspace_bytes(45591, 2944, 2944, 128, 4) == 0


def noalloc_call(T=64, d=256, f=256, E=8, k=2, flags=0, null=None, misalign=None):
    ptrs = [FAKE + 4096 * i for i in range(10)]
    if null is not None:
        ptrs[null] = None
    if misalign is not None:
        ptrs[misalign] += 4
    x, Wr, br, Wgu, Sgu, bgu, Wdn, Sdn, bdn, out = [ctypes.c_void_p(p) if p else None for p in ptrs]
    return moe.lib().moe_forward_noalloc(x, Wr, br, k, Wgu, Sgu, bgu, Wdn, Sdn, bdn, out, T, d, f, E,
                                         flags, None)


@pytest.mark.parametrize("kw,want", [
    (dict(d=200), ERR_SHAPE), (dict(k=9, E=16), ERR_UNSUP), (dict(flags=3), ERR_FLAGS),
    (dict(flags=32), ERR_FLAGS), (dict(null=0), ERR_NULL), (dict(null=9), ERR_NULL),
    (dict(misalign=4), ERR_ALIGN), (dict(T=0, null=0), OK), (dict(T=0, flags=16 | 2), OK),
    # the prefill-shaped layer needs far more than the 64 MiB scratch
    (dict(T=8192, d=2944, f=2944, E=32, k=4), ERR_SCRATCH),
    (dict(T=1026, d=2944, f=2944, E=32, k=4), ERR_SCRATCH),
])
def test_noalloc_argument_errors(kw, want):
    # every case is decided on the host before the scratch is looked up
    assert noalloc_call(**kw) == want


def test_noalloc_scratch_limit_matches_the_workspace_size():
    assert moe.workspace_bytes(1025, 2944, 2944, 32, 4) <= moe.SCRATCH_BYTES
    assert moe.workspace_bytes(1026, 2944, 2944, 32, 4) > moe.SCRATCH_BYTES


def test_gate_options_are_accepted_flags():
    # the routing options are valid bits: with an empty batch the call returns OK
    for fl in (4, 8, 12, 1 | 4, 2 | 8, 1 | 4 | 8):
        assert call(T=0, null=0, flags=fl) == OK
    assert moe.flags_of("decode", "softmax_topk", True) == 2 | 4 | 8
    with pytest.raises(KeyError):
        moe.flags_of(routing="sigmoid")


def test_mx_format_flag_and_entry():
    # MOE_FORMAT_MX is a valid bit on every entry; moe_forward_mx checks like moe_forward_ex
    for fl in (16, 16 | 1, 16 | 2 | 4 | 8, 48, 48 | 2):
        assert call(T=0, null=0, flags=fl) == OK
        assert call(T=0, null=0, flags=fl, stages=(0, 5)) == OK
    assert call(T=0, null=0, entry="mx") == OK
    assert call(T=0, null=0, entry="mx", flags=16) == OK
    assert call(d=200, entry="mx") == ERR_SHAPE
    assert call(null=5, entry="mx") == ERR_NULL
    assert call(flags=3, entry="mx") == ERR_FLAGS
    assert call(ws=100, entry="mx") == ERR_WS
    assert moe.flags_of("prefill", fmt="mx") == 1 | 16
    assert moe.flags_of("decode", fmt="mxfp4") == 2 | 16 | 32
    assert call(T=0, null=0, entry="mx", flags=32) == OK          # FP4 bit: MX is implied by the entry
    assert moe.scale_shapes(256, 384, 8, "mx") == (((8, 8, 768), 1), ((8, 12, 256), 1))
    with pytest.raises(KeyError):
        moe.flags_of(fmt="nvfp4")


def test_empty_batch_is_a_noop():
    assert call(T=0, null=0) == OK          # x may be NULL when T == 0
    assert call(T=0, null=9) == OK          # out may be NULL when T == 0


def test_workspace_size_formula_matches_header_estimate():
    T, d, f, E, k = 4096, 4096, 1536, 128, 8
    est = T * (d + k * (f + 4 * d + 8))
    got = moe.workspace_bytes(T, d, f, E, k)
    assert 0.9 * est < got < 1.2 * est


# ------------------------------------------------------------------ attention with sinks
def attn_prefill_call(S=64, Hq=8, Hkv=2, D=64, null=None, misalign=None):
    ptrs = [FAKE + 4096 * i for i in range(5)]
    if null is not None:
        ptrs[null] = None
    if misalign is not None:
        ptrs[misalign] += 4
    q, k, v, sk, out = [ctypes.c_void_p(p) if p else None for p in ptrs]
    return moe.lib().attn_sink_prefill(q, k, v, sk, out, S, Hq, Hkv, D, 0.125, None)


def attn_decode_call(B=4, Hq=8, Hkv=2, D=64, Lmax=300, ws=None, null=None, misalign=None):
    ptrs = [FAKE + 4096 * i for i in range(7)]
    if null is not None:
        ptrs[null] = None
    if misalign is not None:
        ptrs[misalign] += 4
    q, kc, vc, kl, sk, out, wsp = [ctypes.c_void_p(p) if p else None for p in ptrs]
    if ws is None:
        ws = moe.attn_decode_workspace_bytes(B, Hq, Lmax)
    return moe.lib().attn_sink_decode(q, kc, vc, kl, sk, out, B, Hq, Hkv, D, Lmax, 0.125, wsp, ws, None)


@pytest.mark.parametrize("kw,want", [
    (dict(D=128), ERR_UNSUP), (dict(Hq=6, Hkv=4), ERR_SHAPE), (dict(Hkv=0), ERR_SHAPE), (dict(S=-1), ERR_SHAPE),
    (dict(Hq=24, Hkv=8), ERR_UNSUP), (dict(Hq=12, Hkv=2), ERR_UNSUP), (dict(null=3), ERR_NULL),
    (dict(misalign=0), ERR_ALIGN), (dict(S=0, null=0), OK),
])
def test_attn_prefill_argument_errors(kw, want):
    assert attn_prefill_call(**kw) == want


@pytest.mark.parametrize("kw,want", [
    (dict(D=32), ERR_UNSUP), (dict(Hq=9), ERR_SHAPE), (dict(Hq=64, Hkv=2), ERR_UNSUP), (dict(Lmax=0), ERR_SHAPE),
    (dict(ws=100), ERR_WS), (dict(null=3), ERR_NULL), (dict(null=6), ERR_NULL), (dict(misalign=2), ERR_ALIGN),
    (dict(B=0, null=0), OK),
])
def test_attn_decode_argument_errors(kw, want):
    assert attn_decode_call(**kw) == want


def test_attn_decode_workspace_size():
    # segment records: min(1024 + 2 B, B (ceil(Lmax / 256) + 2)) slots of Hq records of
    # 68 floats, then the plan (2 B + 2 int32, rounded to 16 bytes)
    assert moe.attn_decode_workspace_bytes(4, 8, 256) == 4 * 3 * 8 * 68 * 4 + 48
    assert moe.attn_decode_workspace_bytes(4, 8, 257) == 4 * 4 * 8 * 68 * 4 + 48
    assert moe.attn_decode_workspace_bytes(600, 8, 4096) == (1024 + 1200) * 8 * 68 * 4 + 4816
    assert moe.attn_decode_workspace_bytes(4, 8, 0) == 0
