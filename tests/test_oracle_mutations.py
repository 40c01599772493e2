"""Each test plants one plausible mistake in the oracle (CPU only) and checks
that at least one pin of tests/test_oracle_pins.py then fails."""
import math

import numpy as np
import pytest

from oracle import sks_oracle as orc
from tests import test_oracle_pins as pins
from tests.golden_util import load_examples, load_multi_head_examples

EXAMPLES = load_examples()


def golden_all():
    for ex in EXAMPLES:
        pins.test_golden_worked_examples(ex)


def dense_all():
    for w, k in [(64, 10 ** 6), (1000, 5), (0, 1000)]:
        pins.test_dense_equivalence_against_sdpa(w, k)


def expect_caught(monkeypatch, name, fake, *checks):
    monkeypatch.setattr(orc, name, fake)
    caught = 0
    for chk in checks:
        try:
            chk()
        except AssertionError:
            caught += 1
    assert caught > 0, f"no pin caught the planted mistake in {name}"


def test_caught_tie_break_by_higher_index(monkeypatch):
    def bad(sc, k):
        sc = np.asarray(sc, np.int64)
        order = np.lexsort((-np.arange(sc.shape[0]), -sc))
        return np.sort(order[:min(k, sc.shape[0])])
    expect_caught(monkeypatch, "select_topk", bad, golden_all,
                  lambda: pins.test_topk_brute_force_with_dense_ties(50, 10))


def test_caught_smallest_instead_of_largest(monkeypatch):
    def bad(sc, k):
        sc = np.asarray(sc, np.int64)
        order = np.lexsort((np.arange(sc.shape[0]), sc))
        return np.sort(order[:min(k, sc.shape[0])])
    expect_caught(monkeypatch, "select_topk", bad, golden_all)


def test_caught_wrong_softmax_scale(monkeypatch):
    real = orc.attend
    expect_caught(monkeypatch, "attend", lambda q, K, V, s: real(q, K, V, s / math.sqrt(128)),
                  dense_all)


def test_caught_transposed_value_operand(monkeypatch):
    def bad(q, K, V, s):
        z = (q @ K.T) * s
        p = np.exp(z - z.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        return (p @ K), np.log(np.exp(z).sum(axis=1))      # uses K in place of V
    expect_caught(monkeypatch, "attend", bad, dense_all, golden_all)


def test_caught_dropped_window(monkeypatch):
    def bad(L_i, window, r):
        if L_i <= window:
            return 0, 0
        n_far = (L_i - window) // r
        return n_far, L_i                       # window attended nowhere
    expect_caught(monkeypatch, "row_geometry", bad, golden_all, dense_all)


def test_caught_pool_tail_dropped(monkeypatch):
    def bad(L_i, window, r):
        if L_i <= window:
            return 0, 0
        n_far = (L_i - window) // r
        return n_far, L_i - window              # the < r tail is attended by nobody
    expect_caught(monkeypatch, "row_geometry", bad, golden_all)


def test_caught_pool_without_bf16_rounding(monkeypatch):
    def bad(x, r):
        x = np.asarray(x, np.float64)
        nb = x.shape[0] // r
        return x[: nb * r].reshape(nb, r, x.shape[1]).mean(axis=1)
    expect_caught(monkeypatch, "pool_mean", bad, pins.test_pool_mean_closed_form)


def test_caught_truncating_quantizer(monkeypatch):
    def bad(y, scale):
        return np.clip(np.trunc(np.asarray(y) / scale), -127, 127).astype(np.int8)
    expect_caught(monkeypatch, "quantize_codes", bad,
                  pins.test_key_sketch_coordinate_basis_closed_form, golden_all)


def test_caught_round_half_away_from_zero(monkeypatch):
    def bad(y, scale):
        v = np.asarray(y) / scale
        return np.clip(np.sign(v) * np.floor(np.abs(v) + 0.5), -127, 127).astype(np.int8)
    expect_caught(monkeypatch, "quantize_codes", bad, pins.test_key_sketch_coordinate_basis_closed_form)


def test_caught_projection_with_transposed_basis(monkeypatch):
    def bad(x, basis):
        P = np.asarray(basis, np.float64)
        return np.asarray(x, np.float64)[:, ::-1][:, : P.shape[0]] @ np.eye(P.shape[0])
    expect_caught(monkeypatch, "project", bad, pins.test_key_sketch_coordinate_basis_closed_form,
                  pins.test_key_sketch_orthonormal_projection_invariants)


def test_caught_score_sign_flip(monkeypatch):
    expect_caught(monkeypatch, "scores", lambda qc, kc: -(np.asarray(kc, np.int64) @ np.asarray(qc, np.int64)),
                  golden_all, pins.test_scores_extremes_and_brute_force)


def test_caught_bf16_decode_wrong_shift(monkeypatch):
    def bad(bits):
        u32 = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 15
        return u32.view(np.float32).astype(np.float64)
    expect_caught(monkeypatch, "bf16_to_f64", bad, pins.test_bf16_decode_closed_form)


def test_caught_i4_nibbles_swapped(monkeypatch):
    real = orc.i4_unpack

    def bad(packed):
        p = np.asarray(packed, np.uint8)
        return real(((p << 4) | (p >> 4)).astype(np.uint8))
    expect_caught(monkeypatch, "i4_unpack", bad, pins.test_i4_dequant_hand_decoded)


def test_caught_i4_without_sign_extension(monkeypatch):
    def bad(packed):
        p = np.asarray(packed, np.uint8).astype(np.int64)
        return np.stack([p & 15, p >> 4], axis=-1).reshape(*p.shape[:-1], 2 * p.shape[-1])
    expect_caught(monkeypatch, "i4_unpack", bad, pins.test_i4_dequant_hand_decoded,
                  pins.test_i4_cache_reduces_to_i8_cache_with_the_same_codes)


def test_caught_refit_ascending_order(monkeypatch):
    def bad(G, rank=64):
        w, U = np.linalg.eigh(np.asarray(G, np.float64))
        return U[:, :rank].T.copy(), w
    expect_caught(monkeypatch, "basis_from_gram", bad, pins.test_basis_from_diagonal_gram_closed_form,
                  pins.test_basis_from_planted_gram_and_sign_convention)


def test_caught_refit_without_sign_convention(monkeypatch):
    def bad(G, rank=64):
        w, U = np.linalg.eigh(np.asarray(G, np.float64))
        order = np.argsort(-w, kind="stable")
        return U[:, order][:, :rank].T.copy() * -1.0, w[order]
    expect_caught(monkeypatch, "basis_from_gram", bad, pins.test_basis_from_diagonal_gram_closed_form,
                  pins.test_basis_from_planted_gram_and_sign_convention)


def test_caught_refit_scale_off_by_one(monkeypatch):
    real = orc.project
    expect_caught(monkeypatch, "refit_key_scale",
                  lambda keys, basis: float(np.abs(real(keys, basis)).max()) / 128,
                  pins.test_refit_key_scale_closed_form)



def per_head_goldens():
    for ex in load_multi_head_examples():
        pins.test_golden_per_head_examples(ex)


def test_caught_shared_basis_for_every_head(monkeypatch):
    def bad(basis, h):
        basis = np.asarray(basis, np.float64)
        return basis if basis.ndim == 2 else basis[0]
    expect_caught(monkeypatch, "head_basis", bad, per_head_goldens)


def test_caught_first_head_key_scale_for_every_head(monkeypatch):
    expect_caught(monkeypatch, "head_key_scale",
                  lambda ks, h: float(np.asarray(ks, np.float64)[0]), per_head_goldens)
