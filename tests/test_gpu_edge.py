"""GPU edge cases: the hand-worked examples, degenerate and ragged inputs,
dense equivalence, dense ties, empty rows, verify rows, batch invariance."""
import math

import numpy as np
import pytest
import torch

from long_context_sparse_sketch_amd import binding as sks
from long_context_sparse_sketch_amd import configs as C
from long_context_sparse_sketch_amd.synth import make_case, random_arrays, random_scores
from oracle import sks_oracle as orc
from tests.gpu_util import assert_attn_close, flush, lse_close, run_arrays
from tests.golden_util import (build_inputs, build_multi_head_inputs, load_examples,
                               load_multi_head_examples, parse_value)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("ex", load_examples(), ids=lambda e: e["name"])
def test_golden_worked_examples_on_gpu(ex):
    flush(f"[edge] golden {ex['name']}")
    inp = build_inputs(ex)
    for case in ex["cases"]:
        r = run_arrays(inp["q"], inp["K"], inp["V"], inp["seq_len"], inp["basis"],
                       inp["key_scale"], inp["window"], case["topk"], inp["pool"])
        for i in range(len(ex["q_rows"])):
            n = len(case["scores"][i])
            assert r["scores"][0, i, 0, :n].tolist() == case["scores"][i]
            want_idx = case["idx"][i] + [-1] * (case["topk"] - len(case["idx"][i]))
            assert r["idx"][0, i, 0].tolist() == want_idx
            want = np.zeros(128)
            for d, v in case["out"][i].items():
                want[int(d)] = parse_value(v)
            np.testing.assert_allclose(r["out"][0, i, 0], want, rtol=1e-6, atol=1e-6)
            assert r["lse"][0, i, 0] == pytest.approx(parse_value(case["lse"][i]), rel=1e-6)


@pytest.mark.parametrize("ex", load_multi_head_examples(), ids=lambda e: e["name"])
def test_golden_per_head_examples_on_gpu(ex):
    """One basis and one key scale per KV head (3/8 for head 1, not a power of
    two): codes, scores, indices and outputs as worked out by hand."""
    flush(f"[edge] golden {ex['name']}")
    inp = build_multi_head_inputs(ex)
    for case in ex["cases"]:
        r = run_arrays(inp["q"], inp["K"], inp["V"], inp["seq_len"], inp["basis"],
                       inp["key_scale"], inp["window"], case["topk"], inp["pool"],
                       basis_per_head=True)
        for h in range(ex["Hkv"]):
            assert r["S"][0, h, :, 0].tolist() == ex["key_codes_dim0"][h], h
            assert not r["S"][0, h, :, 1:].any()
            assert r["qsk"][0, 0, h, 0] == ex["qcode_dim0"][h] and not r["qsk"][0, 0, h, 1:].any()
            n = len(case["scores"][h])
            assert r["scores"][0, 0, h, :n].tolist() == case["scores"][h], h
            want_idx = case["idx"][h] + [-1] * (case["topk"] - len(case["idx"][h]))
            assert r["idx"][0, 0, h].tolist() == want_idx, h
            want = np.zeros(128)
            for d, v in case["out"][h].items():
                want[int(d)] = parse_value(v)
            np.testing.assert_allclose(r["out"][0, 0, h], want, rtol=1e-6, atol=1e-6)
            assert r["lse"][0, 0, h] == pytest.approx(parse_value(case["lse"][h]), rel=1e-6)


def oracle_of(q, K, V, Ks, Vs, seq_len, basis, ks, window, topk, pool):
    return orc.decode_step(q, K, V, Ks, Vs, np.asarray(seq_len), basis, ks, window, topk, pool,
                           K.dtype == np.int8)


def compare_all(r, ref, g, R):
    for (b, h), o in ref.items():
        for i in range(R):
            assert np.array_equal(r["idx"][b, i, h], o["idx"][i]), (b, i, h)
            assert r["n_sel"][b, i, h] == o["n_sel"][i]
            sl = slice(h * g, (h + 1) * g)
            assert_attn_close(r["out"][b, i, sl], o["out"][i], f"{(b, i, h)}")
            lse_close(r["lse"][b, i, sl], o["lse"][i], f"{(b, i, h)}")


@pytest.mark.parametrize("window,topk", [(100, 3000), (3000, 5), (0, 2500), (2047, 1),
                                         (100, 1 << 24), (1 << 24, 5)])
def test_dense_and_extreme_selection(window, topk):
    """k >= n_far (dense), window covering all, no window, k = 1, and k at its
    largest (2^24: tens of thousands of attention slots per segment, all but
    the first masked; idx rows padded to 2^24) and the window at its largest."""
    flush(f"[edge] dense/extreme window={window} topk={topk}")
    B, R, Hq, Hkv, T = 2, 1, 8, 2, 2100
    q, K, V, Ks, Vs, basis, ks = random_arrays(B, R, Hq, Hkv, T, seed=window + topk)
    sl = [2048, 1999]
    ref = oracle_of(q, K, V, Ks, Vs, sl, basis, ks, window, topk, 1)
    r = run_arrays(q, K, V, sl, basis, ks, window, topk, ref=ref)
    compare_all(r, ref, Hq // Hkv, R)


@pytest.mark.parametrize("topk", [8192, 8193, 16384, 16385, 20000])
def test_large_k_beyond_register_cache(topk):
    """k at and past the final pass's register slots and LDS cache (8,192
    candidates each): more candidates than they hold take the exact path
    over the candidate lists; with far regions a few times k; two verify
    rows, ragged lengths."""
    flush(f"[edge] large k={topk}")
    B, R, Hq, Hkv, T = 2, 2, 8, 2, 45001
    q, K, V, Ks, Vs, basis, ks = random_arrays(B, R, Hq, Hkv, T, seed=topk)
    sl = [T - R + 1, 30123]
    ref = oracle_of(q, K, V, Ks, Vs, sl, basis, ks, 1000, topk, 1)
    r = run_arrays(q, K, V, sl, basis, ks, 1000, topk, ref=ref)
    compare_all(r, ref, Hq // Hkv, R)


def test_dirty_workspace_with_more_candidates_than_the_lds_cache():
    """A workspace that is not zero at rest makes the final pass's threshold
    guess fail; with more than 8,192 candidates its exact path then runs over
    the candidate lists (not the LDS cache).  Same indices."""
    flush("[edge] dirty workspace, k = 10000")
    B, R, Hq, Hkv, T = 2, 1, 8, 2, 45001
    q, K, V, Ks, Vs, basis, ks = random_arrays(B, R, Hq, Hkv, T, seed=10000)
    sl = [T, 30123]
    ref = oracle_of(q, K, V, Ks, Vs, sl, basis, ks, 1000, 10000, 1)
    r = run_arrays(q, K, V, sl, basis, ks, 1000, 10000, ref=ref)
    compare_all(r, ref, Hq // Hkv, R)
    lay = r["layer"]
    kc = torch.from_numpy(np.stack([np.stack([ref[(b, h)]["kcodes"][:lay.NB] for h in range(Hkv)])
                                    for b in range(B)])).cuda()
    qc = torch.from_numpy(np.stack([np.stack([ref[(b, h)]["qcode"][0] for h in range(Hkv)])
                                    for b in range(B)])[:, None]).cuda()
    for garbage in (0x01010101, 0x00000100):
        lay.ws.view(torch.int32)[: lay.ws.numel() // 4].fill_(garbage)
        lay.score(qsk=qc, S=kc)
        lay.idx.fill_(-7)
        lay.select()
        torch.cuda.synchronize()
        idx = lay.idx.cpu().numpy()
        for (b, h), o in ref.items():
            assert np.array_equal(idx[b, 0, h], o["idx"][0]), (garbage, b, h)


def test_empty_and_short_rows():
    """seq_len 0 (nothing to attend), 1, and shorter than the window."""
    flush("[edge] empty and short rows")
    B, R, Hq, Hkv, T = 4, 1, 4, 1, 600
    q, K, V, Ks, Vs, basis, ks = random_arrays(B, R, Hq, Hkv, T, seed=3)
    sl = [0, 1, 37, 600]
    ref = oracle_of(q, K, V, Ks, Vs, sl, basis, ks, 64, 16, 1)
    r = run_arrays(q, K, V, sl, basis, ks, 64, 16, ref=ref)
    assert not r["out"][0].any() and np.all(np.isneginf(r["lse"][0]))
    assert np.all(r["idx"][0] == -1) and r["n_sel"][0, 0, 0] == 0
    compare_all(r, ref, Hq // Hkv, R)


def test_topk_dense_ties_and_all_equal():
    """Scores from a narrow range (dense ties) and all-equal scores, fed directly."""
    flush("[edge] top-k ties")
    B, R, Hkv, T = 3, 1, 2, 70001
    K = torch.zeros((B, Hkv, T, 128), dtype=torch.bfloat16, device="cuda")
    sl = torch.tensor([T, T, 50000], dtype=torch.int32, device="cuda")
    cache = sks.Cache(K, K, sl)
    W, k = 1000, 2048
    p = sks.params(W, k)
    sc = random_scores((B, R, Hkv, T), -3, 3, seed=17)
    sc[1, 0, 1] = 5                                   # all equal
    sc[2, 0, 0, :20000] = 1000000                     # many maxima
    scores = torch.from_numpy(sc).cuda()
    idx = torch.empty((B, R, Hkv, k), dtype=torch.int32, device="cuda")
    n_sel = torch.empty((B, R, Hkv), dtype=torch.int32, device="cuda")
    ws = torch.empty((sks.workspace_bytes(cache, p, Hkv),), dtype=torch.uint8, device="cuda")
    sks.workspace_init(ws)
    sks.topk_select(scores, cache, p, idx, n_sel, ws)
    got = idx.cpu().numpy()
    for b in range(B):
        n_far = int(sl[b]) - W
        for h in range(Hkv):
            want = orc.pad_idx(orc.select_topk(sc[b, 0, h, :n_far], k), k)
            assert np.array_equal(got[b, 0, h], want), (b, h)
    assert np.array_equal(got[1, 0, 1], np.arange(k))


def test_verify_rows_equal_sequential_on_gpu():
    """R = 3 verify rows give the bits of three R = 1 decodes at L, L+1, L+2."""
    flush("[edge] verify rows")
    cfg = C.small(C.C5)
    case = make_case(cfg, seqs=[0])
    args = (case.K, case.V)
    full = run_arrays(case.q, *args, case.seq_len, case.basis, case.key_scale, cfg.window,
                      cfg.topk, 1, case.K_scale, case.V_scale)
    for i in range(cfg.R):
        one = run_arrays(np.ascontiguousarray(case.q[:, i:i + 1]), *args, case.seq_len + i,
                         case.basis, case.key_scale, cfg.window, cfg.topk, 1, case.K_scale,
                         case.V_scale)
        # the same GPU code computes both: the sketches are identical bits
        assert np.array_equal(full["S"], one["S"])
        assert np.array_equal(full["idx"][:, i], one["idx"][:, 0])
        assert np.array_equal(full["out"][:, i], one["out"][:, 0])
        assert np.array_equal(full["lse"][:, i], one["lse"][:, 0])


@pytest.mark.parametrize("kv", [C.KV_I8, C.KV_BF16], ids=["int8", "bf16"])
def test_verify_rows_in_a_batch_equal_lone_decodes(kv):
    """The workload's own window and top-k, two sequences of three verify
    rows: every row gives the bits of an R = 1 decode of its sequence alone
    at that length, although the batched step has 6x the segments (its
    order of operations may not depend on the batch or the rows)."""
    cfg = C.with_kv(C.full_set(C.C5), kv)
    flush(f"[edge] verify rows in a batch {cfg.name}")
    case = make_case(cfg)
    full = run_arrays(case.q, case.K, case.V, case.seq_len, case.basis, case.key_scale,
                      cfg.window, cfg.topk, 1, case.K_scale, case.V_scale)
    for b in range(cfg.B):
        one = make_case(cfg, seqs=[b])
        for i in range(cfg.R):
            r = run_arrays(np.ascontiguousarray(one.q[:, i:i + 1]), one.K, one.V,
                           one.seq_len + i, one.basis, one.key_scale, cfg.window, cfg.topk, 1,
                           one.K_scale, one.V_scale)
            for key in ("idx", "out", "lse"):
                assert np.array_equal(full[key][b, i], r[key][0, 0]), (b, i, key)


@pytest.mark.parametrize("cfg", [C.small(C.C3), C.small(C.C4)], ids=lambda c: c.name)
def test_batch_invariance_bits(cfg):
    """A sequence gives the same bits alone and inside its batch."""
    flush(f"[edge] batch invariance {cfg.name}")
    full = make_case(cfg)
    one = make_case(cfg, seqs=[1])
    ra = run_arrays(full.q, full.K, full.V, full.seq_len, full.basis, full.key_scale, cfg.window,
                    cfg.topk, cfg.pool)
    rb = run_arrays(one.q, one.K, one.V, one.seq_len, one.basis, one.key_scale, cfg.window,
                    cfg.topk, cfg.pool)
    for key in ("S", "idx", "out", "lse", "qsk"):
        assert np.array_equal(ra[key][1], rb[key][0]), key


def test_ragged_lengths_and_append_mode():
    """Different lengths per sequence; the per-step APPEND sketch of the rows'
    own tokens equals a bulk build over the same positions."""
    flush("[edge] ragged + append")
    cfg = C.small(C.C4)
    case = make_case(cfg)
    sl = np.array([cfg.L, cfg.L - 777], np.int32)
    ref = oracle_of(case.q, case.K, case.V, None, None, sl, case.basis, case.key_scale,
                    cfg.window, cfg.topk, cfg.pool)
    r = run_arrays(case.q, case.K, case.V, sl, case.basis, case.key_scale, cfg.window,
                   cfg.topk, cfg.pool, ref=ref)
    compare_all(r, ref, cfg.g, cfg.R)
    # APPEND: zero the sketch rows of the last block, re-create them with APPEND
    layer = r["layer"]
    S_full = layer.S.clone()
    Kp_full = layer.Kp.clone()
    for b in range(case.B):
        last = (int(sl[b]) - 1) // cfg.pool
        layer.S[b, :, last] = 0
        layer.Kp[b, :, last] = 0
    layer.build_sketch(sks.APPEND, 0)
    torch.cuda.synchronize()
    for b in range(case.B):
        last = (int(sl[b]) - 1) // cfg.pool
        complete = (int(sl[b]) % cfg.pool) == 0
        if complete:
            assert torch.equal(layer.S[b, :, last], S_full[b, :, last])
            assert torch.equal(layer.Kp[b, :, last], Kp_full[b, :, last])
        else:
            assert not layer.S[b, :, last].any()     # block not complete: untouched


def test_bad_arguments_launch_nothing():
    """Invalid arguments return an error code and a message; outputs untouched."""
    K = torch.zeros((1, 1, 64, 128), dtype=torch.bfloat16, device="cuda")
    sl = torch.tensor([64], dtype=torch.int32, device="cuda")
    cache = sks.Cache(K, K, sl)
    out = torch.full((1, 1, 3, 128), 7.0, device="cuda")
    idx = torch.zeros((1, 1, 1, 8), dtype=torch.int32, device="cuda")
    ws = torch.empty((1 << 20,), dtype=torch.uint8, device="cuda")
    q = torch.zeros((1, 1, 3, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(sks.SksError) as e:
        sks.sparse_decode_attn(q, cache, sks.params(8, 8, rank=32), idx, out, ws)
    assert e.value.code == sks.SKS_ERR_ARG and "rank" in str(e.value)
    with pytest.raises(sks.SksError) as e:
        sks.sparse_decode_attn(q, cache, sks.params(8, 8), idx, out, ws[:16])
    assert e.value.code == sks.SKS_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)
