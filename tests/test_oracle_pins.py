"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test fixes a part of the oracle by a closed form, a brute force over tiny
inputs, a library routine it must reduce to, a hand-worked example, or an
invariant the method guarantees.  Method sources: page "8 agents x 250K
context, concurrently, on two 3090s" (claims list; "What it took") and page
"Agens SGLang" README ("What it adds"; "Quick start").
"""
import itertools
import math

import numpy as np
import pytest
import torch

from oracle import sks_oracle as orc
from long_context_sparse_sketch_amd import configs as C
from long_context_sparse_sketch_amd.synth import f32_to_bf16_bits, make_case
from tests.golden_util import (build_inputs, build_multi_head_inputs, load_examples,
                               load_multi_head_examples, parse_value)

SM = 1.0 / math.sqrt(128.0)


# ----------------------------------------------------------------- formats
def test_bf16_decode_closed_form():
    bits = np.array([0x3F80, 0xC000, 0x3F81, 0x0000, 0x8000, 0x7F7F, 0x0001, 0x4049], np.uint16)
    want = [1.0, -2.0, 1.0 + 2.0 ** -7, 0.0, -0.0, (2 - 2.0 ** -7) * 2.0 ** 127, 2.0 ** -133,
            3.140625]
    got = orc.bf16_to_f64(bits)
    assert list(got) == want


def test_f16_decode_closed_form():
    bits = np.array([0x3C00, 0x7BFF, 0x0001, 0xC400, 0x3555], np.uint16)
    want = [1.0, 65504.0, 2.0 ** -24, -4.0, 0.333251953125]
    assert list(orc.f16_to_f64(bits)) == want


def test_i8_dequant_exact():
    codes = np.array([[127, -127, 0, 1]], np.int8)
    scale = np.array([0x3800], np.uint16)     # fp16 0.5
    assert orc.i8_rows_to_f64(codes, scale).tolist() == [[63.5, -63.5, 0.0, 0.5]]


def test_i4_dequant_hand_decoded():
    # bytes 0x21 0xF8 0x07 0x90: low nibble first, two's complement
    #   0x21 -> 1, 2;  0xF8 -> -8, -1;  0x07 -> 7, 0;  0x90 -> 0, -7
    packed = np.array([[0x21, 0xF8, 0x07, 0x90]], np.uint8)
    assert orc.i4_unpack(packed).tolist() == [[1, 2, -8, -1, 7, 0, 0, -7]]
    scale = np.array([0x3800], np.uint16)     # fp16 0.5
    assert orc.i4_rows_to_f64(packed, scale).tolist() == [[0.5, 1.0, -4.0, -0.5, 3.5, 0.0, 0.0,
                                                            -3.5]]
    # every byte value: the two nibbles are (b & 15) and (b >> 4), values >= 8 wrap by 16
    allb = np.arange(256, dtype=np.uint8)[None, :]
    got = orc.i4_unpack(allb)[0]
    for b in range(256):
        lo, hi = b % 16, b // 16
        assert got[2 * b] == (lo if lo < 8 else lo - 16)
        assert got[2 * b + 1] == (hi if hi < 8 else hi - 16)


def test_i4_cache_reduces_to_i8_cache_with_the_same_codes():
    """An int4 cache is an int8 cache whose codes happen to lie in [-8, 7]:
    the whole step must agree exactly with the (separately pinned) int8 path."""
    from long_context_sparse_sketch_amd.synth import pack_i4
    rng = np.random.default_rng(41)
    T, L, Hq, Hkv = 700, 698, 6, 2
    kc = rng.integers(-8, 8, (1, Hkv, T, 128)).astype(np.int8)
    vc = rng.integers(-8, 8, (1, Hkv, T, 128)).astype(np.int8)
    ks = (rng.uniform(0.05, 0.5, (1, Hkv, T))).astype(np.float16).view(np.uint16)
    vs = (rng.uniform(0.05, 0.5, (1, Hkv, T))).astype(np.float16).view(np.uint16)
    q = f32_to_bf16_bits(rng.standard_normal((1, 2, Hq, 128)).astype(np.float32))
    basis = np.linalg.qr(rng.standard_normal((128, 64)))[0].T.astype(np.float32)
    kscale = np.full(Hkv, 1 / 16, np.float32)
    sl = np.array([L], np.int32)
    a = orc.decode_step(q, kc, vc, ks, vs, sl, basis, kscale, 100, 50, 1, orc.KV_I8)
    b = orc.decode_step(q, pack_i4(kc), pack_i4(vc), ks, vs, sl, basis, kscale, 100, 50, 1,
                        orc.KV_I4)
    for key in a:
        for field in ("kcodes",):
            assert np.array_equal(a[key][field], b[key][field])
        for i in range(2):
            for field in ("qcode", "scores", "idx", "out", "lse"):
                assert np.array_equal(a[key][field][i], b[key][field][i]), (key, field, i)


def test_round_to_bf16_ties_and_nearest():
    one = 1.0
    assert orc.round_to_bf16(np.array([one + 2.0 ** -8]))[0] == 1.0                # tie -> even
    assert orc.round_to_bf16(np.array([one + 3 * 2.0 ** -8]))[0] == one + 2.0 ** -6  # tie -> even
    assert orc.round_to_bf16(np.array([one + 2.0 ** -8 + 2.0 ** -30]))[0] == one + 2.0 ** -7
    assert orc.round_to_bf16(np.array([-2.5]))[0] == -2.5
    assert orc.round_to_bf16(np.array([0.0]))[0] == 0.0
    # brute force: the result is a bf16 value no farther from x than its two bf16 neighbours
    rng = np.random.default_rng(7)
    x = rng.standard_normal(2000) * np.exp(rng.uniform(-20, 20, 2000))
    r = orc.round_to_bf16(x)
    bits = orc.f64_to_bf16_bits(r).astype(np.int64)
    assert np.all(orc.bf16_to_f64(bits.astype(np.uint16)) == r)         # exactly representable
    for delta in (-1, 1):
        nb = orc.bf16_to_f64(((bits + delta) & 0xFFFF).astype(np.uint16))
        assert np.all(np.abs(x - r) <= np.abs(x - nb))


# ----------------------------------------------------------------- sketches
def coord_basis():
    P = np.zeros((64, 128))
    P[np.arange(64), np.arange(64)] = 1.0
    return P


def test_key_sketch_coordinate_basis_closed_form():
    k = np.zeros((3, 128))
    k[0, :6] = [1 / 32, 3 / 32, 10.0, -10.0, -5 / 32, 0.7]
    k[1, 64:] = 9.0                                # outside the span: invisible
    k[2, 63] = -7.9375
    y, codes = orc.key_sketch(k, coord_basis(), 1 / 16)
    assert codes[0, :6].tolist() == [0, 2, 127, -127, -2, 11]    # 0.5->0, 1.5->2, clamp, -2.5->-2, 11.2->11
    assert not codes[1].any()
    assert codes[2, 63] == -127                                     # -127.0 exactly
    assert np.array_equal(y[0], k[0, :64])


def test_key_sketch_orthonormal_projection_invariants():
    rng = np.random.default_rng(1)
    P = np.linalg.qr(rng.standard_normal((128, 64)))[0].T
    k = rng.standard_normal((50, 128))
    y, _ = orc.key_sketch(k, P, 1 / 16)
    assert np.all(np.linalg.norm(y, axis=1) <= np.linalg.norm(k, axis=1) + 1e-12)
    c = rng.standard_normal((50, 64))
    y2, _ = orc.key_sketch(c @ P, P, 1 / 16)                   # keys inside span(P)
    np.testing.assert_allclose(y2, c, atol=1e-12)


def test_query_sketch_closed_forms():
    P = coord_basis()
    q = np.zeros((2, 128))
    q[0, 0] = 2.0                                   # group mean = e_0
    codes, scale, _ = orc.query_sketch(q, P)
    assert codes[0] == 127 and not codes[1:].any() and scale == pytest.approx(1 / 127)
    q = np.zeros((1, 128))
    q[0, 0], q[0, 1], q[0, 2], q[0, 70] = -1.0, 0.25, -0.5 - 1 / 254, 5.0
    codes, scale, _ = orc.query_sketch(q, P)
    assert codes[:3].tolist() == [-127, 32, -64]    # 31.75 -> 32; 64.0 -> 64
    assert not codes[3:].any()
    codes, scale, _ = orc.query_sketch(np.zeros((4, 128)), P)
    assert scale == 0.0 and not codes.any()


def test_scores_extremes_and_brute_force():
    q = np.full(64, 127, np.int8)
    k = np.stack([np.full(64, 127), np.full(64, -127), np.zeros(64)]).astype(np.int8)
    assert orc.scores(q, k).tolist() == [1032256, -1032256, 0]
    rng = np.random.default_rng(3)
    q = rng.integers(-127, 128, 64).astype(np.int8)
    k = rng.integers(-127, 128, (20, 64)).astype(np.int8)
    want = [sum(int(a) * int(b) for a, b in zip(q.tolist(), row)) for row in k.tolist()]
    assert orc.scores(q, k).tolist() == want


# ----------------------------------------------------------------- top-k
@pytest.mark.parametrize("n,k", [(1, 1), (7, 3), (50, 10), (200, 64), (4096, 256), (300, 1000)])
def test_topk_brute_force_with_dense_ties(n, k):
    rng = np.random.default_rng(n * 31 + k)
    sc = rng.integers(-3, 4, n)
    sel = orc.select_topk(sc, k)
    want = sorted(i for _, i in sorted((-int(s), i) for i, s in enumerate(sc))[:min(k, n)])
    assert sel.tolist() == want
    k_eff = min(k, n)
    assert sel.shape[0] == k_eff and np.all(np.diff(sel) > 0)
    mask = np.zeros(n, bool)
    mask[sel] = True
    if k_eff < n:
        assert sc[mask].min() >= sc[~mask].max()
        t = sc[mask].min()
        tie_sel, tie_un = np.where(mask & (sc == t))[0], np.where(~mask & (sc == t))[0]
        if tie_un.size:
            assert tie_sel.max() < tie_un.min()


def test_topk_is_best_subset_exhaustive():
    """For tiny n the selection is the k-subset of largest score sum, smallest indices on ties."""
    rng = np.random.default_rng(11)
    for _ in range(30):
        n, k = int(rng.integers(1, 8)), int(rng.integers(1, 8))
        sc = rng.integers(-2, 3, n)
        best = None
        for sub in itertools.combinations(range(n), min(k, n)):
            key = (-sum(int(sc[i]) for i in sub), sub)
            best = key if best is None or key < best else best
        assert orc.select_topk(sc, k).tolist() == list(best[1])


def test_row_geometry_closed_forms():
    assert orc.row_geometry(11, 4, 4) == (1, 4)
    assert orc.row_geometry(13, 4, 4) == (2, 8)
    assert orc.row_geometry(4, 4, 1) == (0, 0)
    assert orc.row_geometry(3, 4, 4) == (0, 0)
    assert orc.row_geometry(250000, 4096, 1) == (245904, 245904)
    assert orc.row_geometry(131072, 4096, 4) == (31744, 126976)
    assert orc.row_geometry(0, 4096, 1) == (0, 0)


def test_pool_mean_closed_form():
    x = np.array([[1.0], [2.0], [3.0], [4.0], [1.0], [1.0], [1.0], [1.0 + 2 ** -7], [9.0]])
    got = orc.pool_mean(x, 4)
    assert got[:, 0].tolist() == [2.5, 1.0]          # 1 + 2^-9 rounds to 1; partial block dropped
    assert np.array_equal(orc.pool_mean(x, 1), x)


# ----------------------------------------------------------------- hand-worked examples
def run_oracle_on(inp, topk):
    return orc.decode_step(inp["q"], inp["K"], inp["V"], None, None, inp["seq_len"], inp["basis"],
                           inp["key_scale"], inp["window"], topk, inp["pool"], False)[(0, 0)]


@pytest.mark.parametrize("ex", load_examples(), ids=lambda e: e["name"])
def test_golden_worked_examples(ex):
    inp = build_inputs(ex)
    for case in ex["cases"]:
        res = run_oracle_on(inp, case["topk"])
        key = "pooled_key_codes_dim0" if ex["pool"] > 1 else "key_codes_dim0"
        assert res["kcodes"][:, 0].tolist() == ex[key]
        assert not res["kcodes"][:, 1:].any()
        for i in range(len(ex["q_rows"])):
            assert res["qcode"][i][0] == ex["qcode_dim0"] and not res["qcode"][i][1:].any()
            assert res["scores"][i].tolist() == case["scores"][i]
            want_idx = case["idx"][i] + [-1] * (case["topk"] - len(case["idx"][i]))
            assert res["idx"][i].tolist() == want_idx
            out = res["out"][i][0]
            want = np.zeros(128)
            for d, v in case["out"][i].items():
                want[int(d)] = parse_value(v)
            np.testing.assert_allclose(out, want, rtol=1e-13, atol=1e-13)
            assert res["lse"][i][0] == pytest.approx(parse_value(case["lse"][i]), rel=1e-13)


@pytest.mark.parametrize("ex", load_multi_head_examples(), ids=lambda e: e["name"])
def test_golden_per_head_examples(ex):
    """One basis and one key scale per KV head (one of them not a power of
    two): every code, score, index, output and lse of each head as worked out
    by hand in the fixture."""
    inp = build_multi_head_inputs(ex)
    for case in ex["cases"]:
        res = orc.decode_step(inp["q"], inp["K"], inp["V"], None, None, inp["seq_len"],
                              inp["basis"], inp["key_scale"], inp["window"], case["topk"],
                              inp["pool"], orc.KV_BF16)
        for h in range(ex["Hkv"]):
            r = res[(0, h)]
            assert r["kcodes"][:, 0].tolist() == ex["key_codes_dim0"][h], h
            assert not r["kcodes"][:, 1:].any()
            assert r["qcode"][0][0] == ex["qcode_dim0"][h] and not r["qcode"][0][1:].any()
            assert r["scores"][0].tolist() == case["scores"][h], h
            want_idx = case["idx"][h] + [-1] * (case["topk"] - len(case["idx"][h]))
            assert r["idx"][0].tolist() == want_idx, h
            want = np.zeros(128)
            for d, v in case["out"][h].items():
                want[int(d)] = parse_value(v)
            np.testing.assert_allclose(r["out"][0][0], want, rtol=1e-13, atol=1e-13)
            assert r["lse"][0][0] == pytest.approx(parse_value(case["lse"][h]), rel=1e-13)


def test_given_codes_reproduce_the_step_and_drive_the_selection():
    """decode_step fed with codes: its own codes give its own results bit for
    bit; codes made by hand select exactly what those codes rank highest."""
    inp = random_inputs(900, 6, 2, 880, seed=17)
    base = orc.decode_step(inp["q"], inp["K"], inp["V"], None, None, inp["seq_len"],
                           inp["basis"], inp["key_scale"], 200, 50, 1, orc.KV_BF16)
    kc = np.stack([base[(0, h)]["kcodes"] for h in range(2)])[None]
    qc = np.stack([base[(0, h)]["qcode"][0] for h in range(2)])[None, None]
    again = orc.decode_step(inp["q"], inp["K"], inp["V"], None, None, inp["seq_len"],
                            inp["basis"], inp["key_scale"], 200, 50, 1, orc.KV_BF16,
                            codes=(kc, qc))
    for key in base:
        for f in ("kcodes", "scores", "idx", "out", "lse"):
            for x, y in zip(np.atleast_1d(base[key][f]), np.atleast_1d(again[key][f])):
                assert np.array_equal(x, y), (key, f)
    # hand-made codes: query e_0 * 1, key t has code t % 97 in dim 0 -> the 50
    # far tokens with the largest t % 97 (ties: lower t) are selected
    kc2 = np.zeros_like(kc)
    kc2[..., 0] = (np.arange(kc.shape[2]) % 97)[None, None, :]
    qc2 = np.zeros_like(qc)
    qc2[..., 0] = 1
    got = orc.decode_step(inp["q"], inp["K"], inp["V"], None, None, inp["seq_len"],
                          inp["basis"], inp["key_scale"], 200, 50, 1, orc.KV_BF16,
                          codes=(kc2, qc2))
    n_far = 880 - 200
    t = np.arange(n_far)
    order = sorted(t, key=lambda x: (-(x % 97), x))[:50]
    for h in range(2):
        assert got[(0, h)]["idx"][0].tolist() == sorted(order)
        assert got[(0, h)]["scores"][0].tolist() == (t % 97).tolist()


# ----------------------------------------------------------------- attention
def random_inputs(T, Hq, Hkv, L, seed, R=1):
    rng = np.random.default_rng(seed)
    return dict(q=f32_to_bf16_bits(rng.standard_normal((1, R, Hq, 128)).astype(np.float32)),
                K=f32_to_bf16_bits(rng.standard_normal((1, Hkv, T, 128)).astype(np.float32)),
                V=f32_to_bf16_bits(rng.standard_normal((1, Hkv, T, 128)).astype(np.float32)),
                basis=np.linalg.qr(rng.standard_normal((128, 64)))[0].T.astype(np.float32),
                key_scale=np.full(Hkv, 1 / 16, np.float32), seq_len=np.array([L], np.int32))


def sdpa_dense(inp, L, row=0):
    """Textbook dense attention via torch's scaled_dot_product_attention (CPU, fp64)."""
    q = torch.from_numpy(orc.bf16_to_f64(inp["q"][0, row]))        # [Hq][D]
    K = torch.from_numpy(orc.bf16_to_f64(inp["K"][0, :, :L]))      # [Hkv][L][D]
    V = torch.from_numpy(orc.bf16_to_f64(inp["V"][0, :, :L]))
    g = q.shape[0] // K.shape[0]
    K, V = K.repeat_interleave(g, 0), V.repeat_interleave(g, 0)
    o = torch.nn.functional.scaled_dot_product_attention(q[:, None, :], K, V, scale=SM)
    return o[:, 0, :].numpy()


@pytest.mark.parametrize("window,topk", [(64, 10 ** 6), (1000, 5), (0, 1000)])
def test_dense_equivalence_against_sdpa(window, topk):
    """Top-k covering every far token (or a window covering all) is dense attention."""
    T, Hq, Hkv, L = 700, 6, 2, 650
    inp = random_inputs(T, Hq, Hkv, L, seed=5)
    res = orc.decode_step(inp["q"], inp["K"], inp["V"], None, None, inp["seq_len"], inp["basis"],
                          inp["key_scale"], window, min(topk, 10 ** 5), 1, False)
    dense = sdpa_dense(inp, L)
    g = Hq // Hkv
    for h in range(Hkv):
        np.testing.assert_allclose(res[(0, h)]["out"][0], dense[h * g:(h + 1) * g], rtol=0, atol=1e-12)


def test_attend_weights_sum_to_one_and_permutation_invariant():
    rng = np.random.default_rng(9)
    q = rng.standard_normal((5, 128))
    K = rng.standard_normal((300, 128)) * 3
    V = np.ones((300, 128))
    out, lse = orc.attend(q, K, V, SM)
    np.testing.assert_allclose(out, 1.0, rtol=0, atol=1e-13)
    V = rng.standard_normal((300, 128))
    out, lse = orc.attend(q, K, V, SM)
    perm = rng.permutation(300)
    out2, lse2 = orc.attend(q, K[perm], V[perm], SM)
    np.testing.assert_allclose(out, out2, atol=1e-13)
    np.testing.assert_allclose(lse, lse2, atol=1e-12)
    z = torch.from_numpy(q) @ torch.from_numpy(K).T * SM
    np.testing.assert_allclose(lse, torch.logsumexp(z, dim=1).numpy(), atol=1e-12)
    out_e, lse_e = orc.attend(q, K[:0], V[:0], SM)
    assert not out_e.any() and np.all(np.isneginf(lse_e))


# ----------------------------------------------------------------- pooling
def test_pool_ratio_one_equals_unpooled_and_repeated_tokens():
    """r = 1 is the unpooled path; r = 4 over a cache of tokens repeated 4x selects
    the same blocks as r = 1 selects tokens of the de-duplicated cache."""
    T, L, W = 400, 400, 40
    inp = random_inputs(T, 4, 2, L, seed=21)
    base = orc.decode_step(inp["q"], inp["K"], inp["V"], None, None, inp["seq_len"], inp["basis"],
                           inp["key_scale"], W, 50, 1, False)
    rep = dict(inp)
    rep["K"] = np.repeat(inp["K"], 4, axis=2)
    rep["V"] = np.repeat(inp["V"], 4, axis=2)
    pooled = orc.decode_step(rep["q"], rep["K"], rep["V"], None, None, np.array([4 * L], np.int32),
                             rep["basis"], rep["key_scale"], 4 * W, 50, 4, False)
    for h in range(2):
        assert np.array_equal(base[(0, h)]["scores"][0], pooled[(0, h)]["scores"][0])
        assert np.array_equal(base[(0, h)]["idx"][0], pooled[(0, h)]["idx"][0])
        assert np.array_equal(base[(0, h)]["kcodes"], pooled[(0, h)]["kcodes"])


def test_pooled_code_is_linear_within_one_lsb():
    rng = np.random.default_rng(4)
    P = np.linalg.qr(rng.standard_normal((128, 64)))[0].T
    x = orc.bf16_to_f64(f32_to_bf16_bits(rng.standard_normal((4000, 128)).astype(np.float32)))
    Kp = orc.pool_mean(x, 4)
    _, codes = orc.key_sketch(Kp, P, 1 / 16)
    ymean = orc.project(x, P).reshape(1000, 4, 64).mean(axis=1)
    lin = np.clip(np.rint(ymean * 16), -127, 127)
    assert np.abs(codes.astype(np.int64) - lin).max() <= 1


# ----------------------------------------------------------------- rows, batches, needles
def test_verify_rows_equal_sequential_decode():
    T, L = 903, 900
    inp = random_inputs(T, 10, 2, L, seed=33, R=3)
    full = orc.decode_step(inp["q"], inp["K"], inp["V"], None, None, inp["seq_len"], inp["basis"],
                           inp["key_scale"], 100, 64, 1, False)
    for i in range(3):
        one = orc.decode_step(inp["q"][:, i:i + 1], inp["K"], inp["V"], None, None,
                              np.array([L + i], np.int32), inp["basis"], inp["key_scale"], 100, 64, 1,
                              False)
        for h in range(2):
            assert np.array_equal(full[(0, h)]["idx"][i], one[(0, h)]["idx"][0])
            np.testing.assert_array_equal(full[(0, h)]["out"][i], one[(0, h)]["out"][0])


def _run_case(case, heads=None):
    cfg = case.cfg
    return orc.decode_step(case.q, case.K, case.V, case.K_scale, case.V_scale, case.seq_len,
                           case.basis, case.key_scale, cfg.window, cfg.topk, cfg.pool,
                           cfg.kv_dtype, heads=heads)


def test_batch_invariance_of_inputs_and_oracle():
    cfg = C.small(C.C5)
    full = make_case(cfg)
    one = make_case(cfg, seqs=[1])
    assert np.array_equal(full.K[1], one.K[0]) and np.array_equal(full.q[1], one.q[0])
    assert np.array_equal(full.K_scale[1], one.K_scale[0])
    a = _run_case(full, heads=[(1, 3)])[(1, 3)]
    b = _run_case(one, heads=[(0, 3)])[(0, 3)]
    for i in range(cfg.R):
        assert np.array_equal(a["idx"][i], b["idx"][i])
        assert np.array_equal(a["out"][i], b["out"][i])


def _check_needles(case, res, row=0):
    cfg = case.cfg
    for (b, h), r in res.items():
        pos = case.needles[(b, h)]
        n_far, ws = r["n_far"][row], r["win_start"][row]
        far = pos[pos < ws]
        units = np.unique(far // cfg.pool)
        sel = r["idx"][row][: r["n_sel"][row]]
        if units.size <= cfg.topk:
            assert np.isin(units, sel).all(), (b, h)
        else:
            assert np.isin(sel, units).all(), (b, h)


@pytest.mark.parametrize("cfg", [C.C1, C.small(C.C2), C.small(C.C3), C.small(C.C4), C.small(C.C5),
                                 C.with_kv(C.small(C.C3), C.KV_I4),
                                 C.with_kv(C.small(C.C5), C.KV_I4)],
                         ids=lambda c: c.name)
def test_needle_recall(cfg):
    case = make_case(cfg)
    heads = [(b, h) for b in range(case.B) for h in range(min(cfg.Hkv, 3))]
    _check_needles(case, _run_case(case, heads))


def test_synth_int8_quantization_bound():
    case = make_case(C.small(C.C5), seqs=[0])
    Kf = orc.i8_rows_to_f64(case.K[0, 0], case.K_scale[0, 0])
    assert np.abs(case.K[0, 0]).max() <= 127
    assert (np.abs(case.K[0, 0]).max(axis=1) >= 126).all()


def test_synth_int4_quantization_bound():
    cfg = C.with_kv(C.small(C.C5), C.KV_I4)
    case = make_case(cfg, seqs=[0])
    assert case.K.shape[-1] == 64 and case.K.dtype == np.uint8
    codes = orc.i4_unpack(case.K[0, 0])
    assert np.abs(codes).max() <= 7 and (np.abs(codes).max(axis=1) == 7).all()
    Kf = orc.i4_rows_to_f64(case.K[0, 0], case.K_scale[0, 0])
    # the int4 rows sit within half a step (plus the fp16 scale's rounding) of the
    # same draw stored as int8, which is itself within half of its own step
    ref = make_case(C.small(C.C5), seqs=[0])
    K8 = orc.i8_rows_to_f64(ref.K[0, 0], ref.K_scale[0, 0])
    s4 = orc.f16_to_f64(case.K_scale[0, 0])[:, None]
    s8 = orc.f16_to_f64(ref.K_scale[0, 0])[:, None]
    assert (np.abs(Kf - K8) <= 0.5 * s4 * 1.01 + 0.5 * s8 + 1e-12).all()


# ----------------------------------------------------------------- basis refit
def test_key_gram_hand_worked_and_brute_force():
    keys = np.zeros((2, 128))
    keys[0, :3] = [1.0, 2.0, 0.5]
    keys[1, :3] = [3.0, -1.0, 0.0]
    G = orc.key_gram(keys)
    # by hand: G00 = 1 + 9, G01 = 2 - 3, G02 = 0.5, G11 = 4 + 1, G12 = 1, G22 = 0.25
    want = np.zeros((128, 128))
    want[:3, :3] = [[10.0, -1.0, 0.5], [-1.0, 5.0, 1.0], [0.5, 1.0, 0.25]]
    assert np.array_equal(G, want)
    rng = np.random.default_rng(5)
    x = rng.standard_normal((37, 128))
    brute = np.zeros((128, 128))
    for row in x:
        for i in range(128):
            brute[i] += row[i] * row
    np.testing.assert_allclose(orc.key_gram(x), brute, rtol=1e-12, atol=1e-12)
    assert orc.key_gram(x).trace() == pytest.approx((x * x).sum(), rel=1e-12)


def test_basis_from_diagonal_gram_closed_form():
    d = np.arange(128, dtype=np.float64)[::-1].copy()        # 127 .. 0
    rng = np.random.default_rng(9)
    perm = rng.permutation(128)
    G = np.diag(d[perm])
    P, w = orc.basis_from_gram(G)
    assert list(w) == sorted(d, reverse=True)
    for r in range(64):
        e = np.zeros(128)
        e[int(np.where(d[perm] == 127 - r)[0][0])] = 1.0       # the r-th largest entry's axis
        assert np.array_equal(P[r], e)


def test_basis_from_planted_gram_and_sign_convention():
    rng = np.random.default_rng(12)
    U = np.linalg.qr(rng.standard_normal((128, 128)))[0]
    lam = np.exp(-np.arange(128) / 20.0)
    G = (U * lam) @ U.T
    P, w = orc.basis_from_gram(G)
    np.testing.assert_allclose(w, lam, rtol=1e-9, atol=1e-14)
    for r in range(64):
        s = 1.0 if np.dot(P[r], U[:, r]) > 0 else -1.0
        np.testing.assert_allclose(P[r], s * U[:, r], atol=1e-8)
        k = int(np.argmax(np.abs(P[r])))
        assert P[r, k] > 0                                       # sign convention
    np.testing.assert_allclose(P @ P.T, np.eye(64), atol=1e-12)
    # rotating G rotates the basis (up to the sign convention)
    Q = np.linalg.qr(rng.standard_normal((128, 128)))[0]
    P2, _ = orc.basis_from_gram(Q @ G @ Q.T)
    for r in range(64):
        v = Q @ P[r]
        assert min(np.abs(P2[r] - v).max(), np.abs(P2[r] + v).max()) < 1e-8


def test_refit_key_scale_closed_form():
    basis = np.eye(128)[:64]
    keys = np.zeros((3, 128))
    keys[0, 5], keys[1, 63], keys[2, 64] = 2.54, -12.7, 99.0   # dim 64 is outside the basis
    assert orc.refit_key_scale(keys, basis) == pytest.approx(12.7 / 127, rel=1e-15)
    assert orc.refit_key_scale(np.zeros((4, 128)), basis) == 1.0


def test_refit_keys_respect_lengths_and_range():
    K = (np.arange(2 * 1 * 10 * 128) % 50).astype(np.uint16).reshape(2, 1, 10, 128) + 0x3F80
    sl = np.array([7, 3], np.int32)
    keys = orc.refit_keys(K, sl, 0, 2, 9)
    assert keys.shape == (5 + 1, 128)                          # [2, 7) of seq 0, [2, 3) of seq 1
    np.testing.assert_array_equal(keys[:5], orc.bf16_to_f64(K[0, 0, 2:7]))
    np.testing.assert_array_equal(keys[5:], orc.bf16_to_f64(K[1, 0, 2:3]))


def test_refit_recovers_planted_subspace():
    from long_context_sparse_sketch_amd.synth import make_refit_keys
    K, U, sigma = make_refit_keys(2, 2, 3000, seed=77)
    sl = np.array([3000, 2500], np.int32)
    G, P, w, scale = orc.refit(K, sl, 0, 3000, per_head=True)
    for h in range(2):
        proj = P[h].T @ P[h]
        truth = U[h][:, :64] @ U[h][:, :64].T
        assert np.abs(proj - truth).max() < 0.05                 # sampling noise only
        keys = orc.refit_keys(K, sl, h, 0, 3000)
        codes = orc.quantize_codes(orc.project(keys, P[h]), scale[h])
        assert np.abs(codes).max() == 127                        # the largest key sits at the edge
    Gs, Ps, _, scale_s = orc.refit(K, sl, 0, 3000, per_head=False)
    np.testing.assert_allclose(Gs[0], G[0] + G[1], rtol=1e-12)

