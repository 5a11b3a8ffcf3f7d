"""Builds the hand-worked block of ``tests/golden/handworked_block.json``.

Inputs are chosen so that every quantisation step is exact (see the fixture's
"inputs" text); the expected outputs there are closed forms derived by hand.
"""
import json
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
FIXTURE = os.path.join(HERE, "golden", "handworked_block.json")


def _bf16(v):
    return (np.asarray(v, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def load():
    with open(FIXTURE) as fh:
        return json.load(fh)


def build(k: int, fmt: str = "block128") -> dict:
    d = f = 128
    E = 2
    x = np.zeros((1, d), np.float32)
    x[0, 0], x[0, 1] = 3.5, 1.75
    Wr = np.zeros((d, E), np.float32)
    Wr[0, 0] = Wr[1, 1] = 1.0
    br = np.zeros(E, np.float32)
    Wgu = np.zeros((E, d, 2 * f), np.uint8)
    Wgu[0, 0, 0], Wgu[0, 1, 0], Wgu[0, 0, f] = 0x38, 0x40, 0x30
    Sgu = np.ones((E, 1, 2), np.float32)
    bgu = np.zeros((E, 2 * f), np.float32)
    bgu[0, f] = 0.25
    Wdn = np.zeros((E, f, d), np.uint8)
    Wdn[0, 0, 0], Wdn[0, 0, 5] = 0x38, 0xB0
    Sdn = np.ones((E, 1, 1), np.float32)
    Sdn[0] = 0.5
    bdn = np.zeros((E, d), np.float32)
    bdn[0, 0], bdn[0, 7] = 0.125, -1.0
    if k == 1:
        Wgu[1] = 0x38
        Wdn[1] = 0x38
    else:
        bdn[1, 3] = 1.0
    if fmt in ("mx", "mxfp4"):  # the same power-of-two scales as E8M0 codes per 32 K rows per column
        Sgu = np.full((E, d // 32, 2 * f), 127, np.uint8)
        Sdn = np.stack([np.full((f // 32, d), 126, np.uint8), np.full((f // 32, d), 127, np.uint8)])
    if fmt == "mxfp4":  # every weight above is an E2M1 value: re-code, pack two per byte along K
        e4m3_to_e2m1 = {0x00: 0x0, 0x38: 0x2, 0x40: 0x4, 0x30: 0x1, 0xB0: 0x9}
        pack = lambda w: (np.vectorize(e4m3_to_e2m1.get)(w[:, 0::2]) |
                          (np.vectorize(e4m3_to_e2m1.get)(w[:, 1::2]) << 4)).astype(np.uint8)
        Wgu, Wdn = pack(Wgu), pack(Wdn)
    return dict(T=1, d=d, d_real=d, f=f, E=E, k=k, x=_bf16(x), W_router=Wr, b_router=br,
                W_gateup=Wgu, S_gateup=Sgu, b_gateup=_bf16(bgu), W_down=Wdn, S_down=Sdn,
                b_down=_bf16(bdn), format=fmt)


def expected(k: int, fmt: str = "block128") -> np.ndarray:
    fx = load()
    exp = fx["mx"]["expected"] if fmt in ("mx", "mxfp4") else fx["expected"]
    out = np.zeros(128)
    for i, v in exp[f"k{k}"].items():
        out[int(i)] = v
    return out
