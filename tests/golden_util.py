"""Loader for the hand-worked fixtures in tests/golden/worked_examples.json."""
import json
import math
import os
from fractions import Fraction

import numpy as np

from long_context_sparse_sketch_amd.synth import f32_to_bf16_bits

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "worked_examples.json")


def load_examples():
    with open(GOLDEN) as f:
        return json.load(f)["examples"]


def parse_value(s):
    """'19/5' -> 3.8, 'ln 5' -> log(5), '1' -> 1.0."""
    s = str(s).strip()
    if s.startswith("ln "):
        return math.log(float(Fraction(s[3:])))
    num, _, den = s.partition("/")
    return float(Fraction(num) / (Fraction(den) if den else 1))


def build_inputs(ex):
    """Arrays (bf16 bit patterns etc.) for one worked example: B = 1, Hq = Hkv = 1."""
    D, rank, T = ex["D"], ex["rank"], ex["T"]
    R = len(ex["q_rows"])
    basis = np.zeros((rank, D), np.float32)
    basis[np.arange(rank), np.arange(rank)] = 1.0
    q = np.zeros((1, R, 1, D), np.float32)
    for i, row in enumerate(ex["q_rows"]):
        for d, v in row.items():
            q[0, i, 0, int(d)] = v
    K = np.zeros((1, 1, T, D), np.float32)
    V = np.zeros((1, 1, T, D), np.float32)
    for t, a in enumerate(ex["a"]):
        K[0, 0, t, 0] = a
        K[0, 0, t, 64] = -a
        V[0, 0, t, 0] = t
        V[0, 0, t, 1] = t * t if "t*t" in ex["V"] else 1.0
    return dict(q=f32_to_bf16_bits(q), K=f32_to_bf16_bits(K), V=f32_to_bf16_bits(V),
                basis=basis, key_scale=np.array([ex["key_scale"]], np.float32),
                seq_len=np.array([ex["L"]], np.int32), window=ex["window"], pool=ex["pool"])


def load_multi_head_examples():
    with open(GOLDEN) as f:
        return json.load(f)["multi_head_examples"]


def build_multi_head_inputs(ex):
    """Arrays for a multi-head worked example: B = 1, one query row, Hq = Hkv,
    one coordinate basis and one key scale per KV head (basis_per_head)."""
    D, rank, T, Hkv = ex["D"], ex["rank"], ex["T"], ex["Hkv"]
    Hq = ex["Hq"]
    basis = np.zeros((Hkv, rank, D), np.float32)
    q = np.zeros((1, 1, Hq, D), np.float32)
    K = np.zeros((1, Hkv, T, D), np.float32)
    V = np.zeros((1, Hkv, T, D), np.float32)
    for h, hd in enumerate(ex["heads"]):
        basis[h, np.arange(rank), hd["basis_start"] + np.arange(rank)] = 1.0
        for d, v in hd["q"].items():
            q[0, 0, h, int(d)] = v
        for t, a in enumerate(hd["a"]):
            K[0, h, t, hd["key_plus_dim"]] = a
            K[0, h, t, hd["key_minus_dim"]] = -a
            V[0, h, t, 0] = t
            V[0, h, t, 1] = t * t
    return dict(q=f32_to_bf16_bits(q), K=f32_to_bf16_bits(K), V=f32_to_bf16_bits(V),
                basis=basis, key_scale=np.array([hd["key_scale"] for hd in ex["heads"]], np.float32),
                seq_len=np.array([ex["L"]], np.int32), window=ex["window"], pool=ex["pool"])
