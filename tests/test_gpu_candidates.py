"""GPU parity of the selection's candidate mode (sks_score_candidates +
sks_topk_select_candidates, and sks_decode_step with SKS_STEP_NO_SCORES),
through the C ABI, against the oracle's selection.

The estimate E that decides which far entries are kept only changes the time
taken, so each case runs with the sample pass's estimate and with the two
forced ones: above every key (every segment recomputes its scores from the
sketches) and zero (every far entry is a candidate).  A workspace holding
garbage (estimates and histograms) must give the same indices.  The fused
step without stored scores must give the stored-score step's indices,
outputs and log-sum-exps bit for bit.
"""
import numpy as np
import pytest
import torch

from long_context_sparse_sketch_amd import binding as sks
from long_context_sparse_sketch_amd import configs as C
from long_context_sparse_sketch_amd.synth import make_case
from tests.gpu_util import GpuCase, flush, ref_arrays
from tests.test_gpu_parity import CFGS
from tests.test_gpu_random_shapes import draw

pytestmark = pytest.mark.gpu

MODES = {"sampled": 0, "high": sks.CAND_TEST_HIGH, "zero": sks.CAND_TEST_ZERO}


@pytest.fixture(scope="module", params=CFGS, ids=lambda c: c.name)
def ctx(request):
    cfg = request.param
    flush(f"[candidates] case {cfg.name}: generating + oracle")
    case = make_case(cfg)
    g = GpuCase(case)
    ref = g.oracle()
    arr = ref_arrays(ref, cfg, case.B, g.topk, g.layer.NB)
    flush(f"[candidates] case {cfg.name}: GPU full step")
    g.run_full()
    return cfg, case, g, ref, arr


def select_candidates(g, arr, flags):
    """Candidate mode on the oracle's codes; returns (idx, n_sel) on the host."""
    qc = torch.from_numpy(arr["qcode"]).cuda()
    kc = torch.from_numpy(arr["kcodes"]).cuda()
    g.layer.score_candidates(qsk=qc, S=kc, flags=flags)
    g.layer.idx.fill_(-7)
    g.layer.n_sel.fill_(-7)
    g.layer.select_candidates(qsk=qc, S=kc)
    torch.cuda.synchronize()
    return g.layer.idx.cpu().numpy(), g.layer.n_sel.cpu().numpy()


@pytest.mark.parametrize("mode", list(MODES))
def test_candidates_given_oracle_codes(ctx, mode):
    cfg, case, g, ref, arr = ctx
    idx, n_sel = select_candidates(g, arr, MODES[mode])
    assert np.array_equal(idx, arr["idx"]), (cfg.name, mode)
    assert np.array_equal(n_sel, arr["n_sel"]), (cfg.name, mode)


def test_candidates_with_dirty_workspace(ctx):
    """Garbage estimates and histograms cost time, never correctness."""
    cfg, case, g, ref, arr = ctx
    qc = torch.from_numpy(arr["qcode"]).cuda()
    kc = torch.from_numpy(arr["kcodes"]).cuda()
    for garbage in (0x01010101, -1, 0x7fffffff, 0x00100000, 0):
        g.layer.ws.view(torch.int32)[: g.layer.ws.numel() // 4].fill_(garbage)
        g.layer.score_candidates(qsk=qc, S=kc, flags=sks.CAND_KEEP_ESTIMATE)
        g.layer.idx.fill_(-7)
        g.layer.select_candidates(qsk=qc, S=kc)
        torch.cuda.synchronize()
        assert np.array_equal(g.layer.idx.cpu().numpy(), arr["idx"]), (cfg.name, garbage)
    sks.workspace_init(g.layer.ws)
    idx, _ = select_candidates(g, arr, 0)
    assert np.array_equal(idx, arr["idx"])


def test_step_without_scores_equals_step(ctx):
    """SKS_STEP_NO_SCORES: the same idx, n_sel, out and lse bit for bit
    (rows of more than 8,192 far entries take the candidate mode: at 65,536
    far entries per row or fewer, or single rows with 2^20 far entries in
    all; the others store the scores as before)."""
    cfg, case, g, ref, arr = ctx
    lay = g.layer
    lay.step(g.q)
    torch.cuda.synchronize()
    want = [t.clone() for t in (lay.idx, lay.n_sel, lay.out, lay.lse)]
    for t in (lay.idx, lay.n_sel):
        t.fill_(-7)
    lay.out.fill_(float("nan"))
    lay.lse.fill_(float("nan"))
    lay.step(g.q, keep_scores=False)
    torch.cuda.synchronize()
    for name, a, b in zip(("idx", "n_sel", "out", "lse"), want,
                          (lay.idx, lay.n_sel, lay.out, lay.lse)):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32)), (cfg.name, name)


def histogram_regions(lay):
    """The per-segment histograms at the start of the workspace that must be
    zero at rest: level-1, level-2 and the sample histograms (the layout of
    the selection's workspace: level-1 [nseg][2048], level-2 [nseg][1024],
    thresholds [nseg][4], sub-list maxima [nseg][ceil(NB / 1024)], sample
    [nseg][2048] int32, each region 256-byte aligned)."""
    def align(x):
        return (x + 255) // 256 * 256
    nseg = lay.B * lay.R * lay.Hkv
    n_sub = (lay.NB + 1023) // 1024
    h1, h2 = nseg * 2048 * 4, nseg * 1024 * 4
    samp = align(h1) + align(h2) + align(nseg * 16) + align(nseg * n_sub * 4)
    ws = lay.ws
    return {"level-1": ws[:h1], "level-2": ws[align(h1):align(h1) + h2], "sample": ws[samp:samp + h1]}


def test_histograms_return_to_zero(ctx):
    """After the candidate selection and after a step (in candidate mode for
    the shapes that take it: the attention's merge launch clears the sample
    histograms there), every histogram of the workspace is zero again, so
    that the next selection's estimate and thresholds start clean."""
    cfg, case, g, ref, arr = ctx
    lay = g.layer
    sks.workspace_init(lay.ws)
    select_candidates(g, arr, 0)
    for name, r in histogram_regions(lay).items():
        assert int(torch.count_nonzero(r)) == 0, (cfg.name, "candidate selection", name)
    for keep in (False, True, False):
        lay.step(g.q, keep_scores=keep)
        torch.cuda.synchronize()
        for name, r in histogram_regions(lay).items():
            assert int(torch.count_nonzero(r)) == 0, (cfg.name, "step", keep, name)


@pytest.mark.parametrize("seed", list(range(60)))
def test_candidates_random_shape(seed):
    """Ragged lengths (empty rows included), verify rows, pooling, k = 1 and
    window 0, as the random-shape parity draws them, in all three modes."""
    cfg, sl = draw(seed)
    flush(f"[candidates random] seed {seed}: B={cfg.B} R={cfg.R} Hkv={cfg.Hkv} L={sl.tolist()} "
          f"W={cfg.window} k={cfg.topk} r={cfg.pool}")
    case = make_case(cfg)
    g = GpuCase(case, seq_len=sl)
    ref = g.oracle()
    arr = ref_arrays(ref, cfg, case.B, g.topk, g.layer.NB)
    for mode, flags in MODES.items():
        idx, n_sel = select_candidates(g, arr, flags)
        assert np.array_equal(idx, arr["idx"]), (seed, mode)
        assert np.array_equal(n_sel, arr["n_sel"]), (seed, mode)


def test_step_in_candidate_mode_clears_histograms():
    """A shape that takes candidate mode in the step (one row, 8 segments of
    ~136K far entries: more than 2^20 in all): the step without scores gives
    the stored-score step's bits, and after each such step every histogram of
    the workspace is zero again (the sample histograms are cleared by the
    attention's merge launch there)."""
    cfg = C.C3.scaled(name="candidate_step", B=2, L=140000, needle_count=16)
    flush(f"[candidates] {cfg.name}: B={cfg.B} Hkv={cfg.Hkv} L={cfg.L}")
    case = make_case(cfg)
    g = GpuCase(case)
    lay = g.layer
    lay.build_sketch(0, g.T)
    lay.step(g.q)
    torch.cuda.synchronize()
    want = [t.clone() for t in (lay.idx, lay.n_sel, lay.out, lay.lse)]
    for _ in range(3):
        for t in (lay.idx, lay.n_sel):
            t.fill_(-7)
        lay.out.fill_(float("nan"))
        lay.step(g.q, keep_scores=False)
        torch.cuda.synchronize()
        for name, a, b in zip(("idx", "n_sel", "out", "lse"), want,
                              (lay.idx, lay.n_sel, lay.out, lay.lse)):
            assert torch.equal(a.view(torch.int32), b.view(torch.int32)), name
        for name, r in histogram_regions(lay).items():
            assert int(torch.count_nonzero(r)) == 0, name
