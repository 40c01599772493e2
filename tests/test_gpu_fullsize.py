"""Parity at the full workload sizes, in the launch configuration the
benchmark times (the step captured in a HIP graph and replayed), on sampled
segments that the oracle computes one by one.

For each configuration:
* the GPU key sketch of sampled (sequence, KV head) pairs meets the sketch
  bound against the oracle's float64 projection;
* with the oracle's int8 key/query codes written into the sampled segments,
  the GPU scores and selected indices there are bit-exact and the attention
  outputs are within tolerance (same kernels and launch shapes as the graph);
* the selection's candidate mode gives the same indices there, with the
  sample pass's estimate and with every segment recomputing its scores;
* the end-to-end step (GPU sketches) recalls the planted needles on every
  segment of the batch;
* the step without stored scores (candidate mode, as the benchmark runs it)
  gives the stored-score step's indices, outputs and log-sum-exps bit for
  bit on every segment.
"""
import numpy as np
import pytest
import torch

from long_context_sparse_sketch_amd import binding as sks
from long_context_sparse_sketch_amd import configs as C
from long_context_sparse_sketch_amd.runtime import StepRunner
from long_context_sparse_sketch_amd.synth import make_case
from oracle import sks_oracle as orc
from tests.gpu_util import GpuCase, assert_attn_close, flush, lse_close, sketch_ok

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


def sample_pairs(cfg):
    B, H = cfg.B, cfg.Hkv
    return sorted({(0, 0), (B - 1, H - 1), (B // 2, H // 2)})


@pytest.mark.parametrize("cfg", [C.C2, C.C3, C.C4, C.C5, C.with_kv(C.C3, C.KV_I4),
                                 C.with_kv(C.C3, C.KV_I8)],
                         ids=lambda c: c.name)
def test_full_size_sampled_parity(cfg):
    flush(f"[full] {cfg.name}: generating {cfg.B} x {cfg.L}")
    case = make_case(cfg)
    g = GpuCase(case)
    runner = StepRunner(g.layer)
    g.layer.build_sketch(0, g.T)
    runner.capture(g.q)
    runner.replay()
    torch.cuda.synchronize()
    pairs = sample_pairs(cfg)
    flush(f"[full] {cfg.name}: oracle on {pairs}")
    ref = g.oracle(heads=pairs)

    # 1. GPU key sketches of the sampled pairs
    S = g.layer.S
    for (b, h), r in ref.items():
        Kf, _ = orc.cache_rows(case.K, case.V, case.K_scale, case.V_scale, b, h,
                               cfg.kv_dtype)
        y = orc.project(orc.pool_mean(Kf, cfg.pool), case.basis)[: g.layer.NB]
        got = S[b, h].cpu().numpy()
        assert sketch_ok(got, y, float(case.key_scale[h])).all(), (b, h)

    # 2. the same kernels and launch shapes on the oracle's int8 codes, written
    #    into the sampled segments (segments never interact): bit-exact scores
    #    and indices, attention within tolerance
    for (b, h), r in ref.items():
        g.layer.S[b, h].copy_(torch.from_numpy(r["kcodes"][: g.layer.NB]))
        for i in range(cfg.R):
            g.layer.qsk[b, i, h].copy_(torch.from_numpy(r["qcode"][i]))
    g.layer.score()
    g.layer.select()
    g.layer.attend(g.q)
    torch.cuda.synchronize()
    scores = g.layer.scores.cpu().numpy()
    idx = g.layer.idx.cpu().numpy()
    out = g.layer.out.cpu().numpy()
    lse = g.layer.lse.cpu().numpy()
    gq = cfg.g
    for (b, h), r in ref.items():
        for i in range(cfg.R):
            n = len(r["scores"][i])
            assert np.array_equal(scores[b, i, h, :n], r["scores"][i]), (b, i, h)
            assert np.array_equal(idx[b, i, h], r["idx"][i]), (b, i, h)
            sl = slice(h * gq, (h + 1) * gq)
            assert_attn_close(out[b, i, sl], r["out"][i], f"{cfg.name} {(b, i, h)}")
            lse_close(lse[b, i, sl], r["lse"][i], f"{cfg.name} {(b, i, h)}")

    # 2b. the selection's candidate mode on the same codes: the same indices,
    #     with the sample pass's estimate and with every segment recomputing
    qc, kc = g.layer.qsk.clone(), g.layer.S
    for flags in (0, sks.CAND_TEST_HIGH):
        g.layer.score_candidates(qsk=qc, S=kc, flags=flags)
        g.layer.idx.fill_(-7)
        g.layer.select_candidates(qsk=qc, S=kc)
        torch.cuda.synchronize()
        idx = g.layer.idx.cpu().numpy()
        for (b, h), r in ref.items():
            for i in range(cfg.R):
                assert np.array_equal(idx[b, i, h], r["idx"][i]), (flags, b, i, h)

    # 3. end to end (GPU sketches, graph replay): on the sampled pairs, the
    #    oracle's scores, selection and attention on the GPU's own codes give
    #    the same indices and outputs within tolerance; needle recall on every
    #    segment
    g.layer.build_sketch(0, g.T)
    runner.replay()
    torch.cuda.synchronize()
    idx = g.layer.idx.cpu().numpy()
    n_sel = g.layer.n_sel.cpu().numpy()
    out = g.layer.out.cpu().numpy()
    lse = g.layer.lse.cpu().numpy()
    Sg, qg = g.layer.S.cpu().numpy(), g.layer.qsk.cpu().numpy()
    ref_own = g.oracle(heads=pairs, codes=(Sg, qg))
    for (b, h), r in ref_own.items():
        for i in range(cfg.R):
            assert np.array_equal(idx[b, i, h], r["idx"][i]), ("own codes", b, i, h)
            assert n_sel[b, i, h] == r["n_sel"][i]
            sl = slice(h * gq, (h + 1) * gq)
            assert_attn_close(out[b, i, sl], r["out"][i], f"{cfg.name} own codes {(b, i, h)}")
            lse_close(lse[b, i, sl], r["lse"][i], f"{cfg.name} own codes {(b, i, h)}")
    for (b, h), pos in case.needles.items():
        Li = int(case.seq_len[b])
        n_far, ws = orc.row_geometry(Li, cfg.window, cfg.pool)
        units = np.unique(pos[pos < ws] // cfg.pool)
        sel = idx[b, 0, h, : n_sel[b, 0, h]]
        if units.size <= cfg.topk:
            assert np.isin(units, sel).all(), (b, h)
        else:
            assert np.isin(sel, units).all(), (b, h)

    # 4. the benchmark's step (SKS_STEP_NO_SCORES: candidate mode at these
    #    sizes) against the stored-score step, every segment, bit for bit
    lay = g.layer
    want = [t.clone() for t in (lay.idx, lay.n_sel, lay.out, lay.lse)]
    runner_ns = StepRunner(lay, keep_scores=False)
    runner_ns.capture(g.q)
    for t in (lay.idx, lay.n_sel):
        t.fill_(-7)
    runner_ns.replay()
    torch.cuda.synchronize()
    for name, a, b in zip(("idx", "n_sel", "out", "lse"), want,
                          (lay.idx, lay.n_sel, lay.out, lay.lse)):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32)), (cfg.name, name)
    flush(f"[full] {cfg.name}: ok")
