"""GPU parity of whole decode steps on seeded random long-context shapes that
take the selection's candidate mode when they store no scores: far regions of
8K to 320K entries per row and at least 2^20 in all (the estimate from the
sample histograms, single-row steps), and far regions of 8,193 to 65,536
entries per row with one to three verify rows (the estimate from one sample
workgroup per segment)
("What it took" on the page "8 agents x 250K context, concurrently, on two
3090s": score every token, pick the top ~2K).  Each case draws the batch, the
verify rows, the query group, pooling, KV storage, window, top-k (up to
12,000) and the needle layout (scattered, or 1% of the tokens in 8 clusters),
with ragged lengths: one full-length row, others random, a row short enough
that its top-k takes every far entry, an empty row.

Per case, through the C ABI:
* the step without stored scores equals the step with them, bit for bit
  (idx, n_sel, out, lse), twice in a row;
* every selection histogram of the workspace is zero again afterwards;
* on sampled (sequence, KV head) pairs, idx and n_sel equal the oracle's
  selection from the GPU's own sketches, and out and lse are within the
  output bound of the oracle's attention over that selection.
"""
import numpy as np
import pytest
import torch

from long_context_sparse_sketch_amd import configs as C
from long_context_sparse_sketch_amd.synth import make_case
from tests.gpu_util import GpuCase, assert_attn_close, flush, lse_close
from tests.test_gpu_candidates import histogram_regions

pytestmark = pytest.mark.gpu

SEEDS = list(range(40))
EST_SEEDS = list(range(24))


def draw(seed):
    rng = np.random.default_rng(91000 + seed)
    while True:
        R = int(rng.choice([1, 1, 1, 1, 2, 3]))
        Hkv = int(rng.integers(1, 5))
        G = int(rng.integers(1, 9))
        pool = int(rng.choice([1, 1, 1, 2, 4]))
        kv = C.KV_BF16 if pool > 1 else int(rng.choice([C.KV_BF16, C.KV_I8, C.KV_I4]))
        window = int(rng.choice([0, 17, 4096, int(rng.integers(0, 6000))]))
        topk = int(rng.choice([1, 3, 2048, int(rng.integers(1, 12000))]))
        B = int(rng.integers(1, 5))
        nseg = B * R * Hkv
        # the step's candidate mode: more than 8,192 far entries per row and
        # at least 2^20 over the batch's segments
        need_far = max(8193, -(-(1 << 20) // nseg))
        L_min = window + pool * need_far + 1
        L = int(rng.integers(L_min, L_min + 60000))
        if L <= 320000:
            break
    kind = str(rng.choice(["random", "clusters"]))
    cfg = C.Config(f"long{seed}", 300 + seed, B=B, R=R, Hq=Hkv * G, Hkv=Hkv, L=L, window=window,
                   topk=topk, pool=pool, kv_dtype=kv, needle_kind=kind,
                   needle_count=(L // 100 if kind == "clusters" else 64), needle_amp=2.5,
                   needle_noise=0.5)
    lengths = rng.integers(0, L + 1, B).astype(np.int32)
    lengths[0] = L
    if B > 1 and rng.random() < 0.4:
        lengths[1] = int(rng.integers(0, window + topk + 2))
    if B > 2 and rng.random() < 0.4:
        lengths[2] = 0
    return cfg, lengths


def draw_early(seed):
    rng = np.random.default_rng(77000 + seed)
    R = int(rng.choice([1, 1, 2, 3, 3]))
    Hkv = int(rng.integers(1, 9))
    G = int(rng.integers(1, 9))
    pool = int(rng.choice([1, 1, 1, 2, 4]))
    kv = C.KV_BF16 if pool > 1 else int(rng.choice([C.KV_BF16, C.KV_I8, C.KV_I4]))
    window = int(rng.choice([0, 17, 4096, int(rng.integers(0, 6000))]))
    topk = int(rng.choice([1, 3, 2048, int(rng.integers(1, 8000))]))
    B = int(rng.integers(1, 7))
    far = int(rng.integers(8193, 65537))        # far entries of a full-length row
    L = window + pool * far + R
    kind = str(rng.choice(["random", "clusters"]))
    cfg = C.Config(f"early{seed}", 500 + seed, B=B, R=R, Hq=Hkv * G, Hkv=Hkv, L=L, window=window,
                   topk=topk, pool=pool, kv_dtype=kv, needle_kind=kind,
                   needle_count=(L // 100 if kind == "clusters" else 64), needle_amp=2.5,
                   needle_noise=0.5)
    lengths = rng.integers(0, L + 1, B).astype(np.int32)
    lengths[0] = L
    if B > 1 and rng.random() < 0.4:
        lengths[1] = int(rng.integers(0, window + topk + 2))
    if B > 2 and rng.random() < 0.4:
        lengths[2] = 0
    return cfg, lengths


@pytest.mark.parametrize("seed", SEEDS)
def test_long_random_step(seed):
    check_step(seed, *draw(seed))


@pytest.mark.parametrize("seed", EST_SEEDS)
def test_early_estimate_random_step(seed):
    check_step(seed, *draw_early(seed))


def check_step(seed, cfg, sl):
    flush(f"[long random] {cfg.name}: B={cfg.B} R={cfg.R} Hq/Hkv={cfg.Hq}/{cfg.Hkv} "
          f"L={sl.tolist()} W={cfg.window} k={cfg.topk} r={cfg.pool} "
          f"kv={C.KV_NAMES[cfg.kv_dtype]} needles={cfg.needle_kind}")
    case = make_case(cfg)
    g = GpuCase(case, seq_len=sl)
    lay = g.layer
    lay.build_sketch(0, g.T)
    lay.step(g.q)
    torch.cuda.synchronize()
    want = [t.clone() for t in (lay.idx, lay.n_sel, lay.out, lay.lse)]
    for rep in range(2):
        for t in (lay.idx, lay.n_sel):
            t.fill_(-7)
        lay.out.fill_(float("nan"))
        lay.lse.fill_(float("nan"))
        lay.step(g.q, keep_scores=False)
        torch.cuda.synchronize()
        for name, a, b in zip(("idx", "n_sel", "out", "lse"), want,
                              (lay.idx, lay.n_sel, lay.out, lay.lse)):
            assert torch.equal(a.view(torch.int32), b.view(torch.int32)), (seed, rep, name)
    for name, r in histogram_regions(lay).items():
        assert int(torch.count_nonzero(r)) == 0, (seed, name)

    kc = lay.S.cpu().numpy()
    qc = lay.qsk.cpu().numpy()
    rng = np.random.default_rng(seed)
    pairs = {(0, 0), (cfg.B - 1, cfg.Hkv - 1)}
    while len(pairs) < min(4, cfg.B * cfg.Hkv):
        pairs.add((int(rng.integers(0, cfg.B)), int(rng.integers(0, cfg.Hkv))))
    ref = g.oracle(heads=sorted(pairs), codes=(kc, qc))
    idx = lay.idx.cpu().numpy()
    n_sel = lay.n_sel.cpu().numpy()
    out = lay.out.cpu().numpy()
    lse = lay.lse.cpu().numpy()
    G = cfg.g
    for (b, h), r in ref.items():
        for i in range(cfg.R):
            assert np.array_equal(idx[b, i, h], r["idx"][i]), (seed, b, i, h)
            assert n_sel[b, i, h] == r["n_sel"][i], (seed, b, i, h)
            assert_attn_close(out[b, i, h * G:(h + 1) * G], r["out"][i], f"{seed} {b} {i} {h}")
            lse_close(lse[b, i, h * G:(h + 1) * G], r["lse"][i], f"{seed} {b} {i} {h}")
