"""The largest sizes the library supports.

test_largest_cache -- the largest cache the selection supports: one sequence of 8,388,608
tokens per KV head (T_max / pool at the limit: 8,192 sub-lists of 1,024
sketch rows in the final pass), two KV heads, through the whole step (bulk
key sketch, then sks_decode_step), against the oracle, for each head:

* key sketch codes on a sample of 65,536 positions (and both ends) within
  the sketch bound, the query sketch likewise;
* every far token's score (8,384,512 of them) bit-exact given the GPU's codes;
* the selected indices bit-exact (the oracle's full sort of all scores);
* the attention output within the output bound, over the oracle's rows;
* the selection's candidate mode (131,008 sampled rows per head, 256 sample
  workgroups each) picks the same indices, with the sampled estimate and
  with every head recomputing its scores.

The second head's K and V rows lie 2 GiB and more past the start of the
cache, so every byte offset into it needs 64-bit arithmetic."""
import math

import numpy as np
import pytest
import torch

from long_context_sparse_sketch_amd import binding as sks
from long_context_sparse_sketch_amd import configs as C
from long_context_sparse_sketch_amd.runtime import SparseDecodeLayer
from long_context_sparse_sketch_amd.synth import make_case_on_device
from oracle import sks_oracle as orc
from tests.gpu_util import assert_attn_close, flush, lse_close, sketch_ok

pytestmark = pytest.mark.gpu

MAX_ROWS = 8192 * 1024        # sketch rows (T_max / pool) the selection supports
WINDOW, TOPK, HKV, G = 4096, 2048, 2, 4


def rows_f64(t, pos):
    """bf16 rows t[pos] of a device tensor [T][128] as float64 on the host."""
    idx = torch.from_numpy(np.asarray(pos, np.int64)).to(t.device)
    return orc.bf16_to_f64(t[idx].view(torch.int16).cpu().numpy().view(np.uint16))


def test_largest_cache():
    L = MAX_ROWS
    cfg = C.Config("max_cache", 91, B=1, R=1, Hq=HKV * G, Hkv=HKV, L=L, window=WINDOW,
                   topk=TOPK, pool=1, kv_dtype=C.KV_BF16, needle_kind="random",
                   needle_count=64, needle_amp=3.0, needle_noise=0.5)
    assert cfg.T_max == MAX_ROWS
    flush(f"[max] drawing {HKV} x {L} tokens on the device")
    case = make_case_on_device(cfg, "cuda")
    K, V = case.K, case.V
    sl = torch.from_numpy(case.seq_len.copy()).cuda()
    cache = sks.Cache(K, V, sl)
    layer = SparseDecodeLayer(1, 1, HKV * G, HKV, cfg.T_max, WINDOW, TOPK, 1, sks.KV_BF16)
    layer.bind(cache, torch.from_numpy(case.basis).cuda(), torch.from_numpy(case.key_scale).cuda())
    q = torch.from_numpy(case.q.view(np.int16)).cuda().view(torch.bfloat16)
    flush("[max] bulk sketch + step")
    layer.build_sketch(0, cfg.T_max)
    layer.step(q)
    torch.cuda.synchronize()
    n_far = L - WINDOW
    qf_all = orc.bf16_to_f64(case.q[0, 0])
    rng = np.random.default_rng(5)
    for h in range(HKV):
        flush(f"[max] KV head {h}: sketches")
        # sketches: a seeded sample of positions and both ends
        pos = np.unique(np.concatenate([rng.integers(0, L, 65536), np.arange(16),
                                        np.arange(L - 16, L)]))
        y = orc.project(rows_f64(K[0, h], pos), case.basis)
        S = layer.S[0, h]
        got = S[torch.from_numpy(pos).cuda()].cpu().numpy()
        assert sketch_ok(got, y, float(case.key_scale[h])).all()
        qf = qf_all[h * G:(h + 1) * G]
        _, qs, yq = orc.query_sketch(qf, case.basis)
        qc = layer.qsk[0, 0, h].cpu().numpy()
        assert sketch_ok(qc, yq, qs).all()

        # every score, given the GPU's codes
        flush(f"[max] KV head {h}: oracle scores of every far token")
        codes = S[:n_far].cpu().numpy()
        chunk = 1 << 20
        ref = np.concatenate([orc.scores(qc, codes[c:c + chunk]) for c in range(0, n_far, chunk)])
        del codes
        assert np.array_equal(layer.scores[0, 0, h, :n_far].cpu().numpy().astype(np.int64), ref)

        # selection: the oracle's full sort
        flush(f"[max] KV head {h}: oracle selection")
        sel = orc.select_topk(ref, TOPK)
        assert np.array_equal(layer.idx[0, 0, h].cpu().numpy(), sel.astype(np.int32))
        assert int(layer.n_sel[0, 0, h]) == TOPK
        needles = case.needles[(0, h)]
        flush(f"[max] KV head {h}: needles kept {np.isin(needles, sel).sum()} / {needles.size}")

        # attention over the selected rows and the window
        rows = np.concatenate([sel, np.arange(n_far, L)])
        out, lse = orc.attend(qf, rows_f64(K[0, h], rows), rows_f64(V[0, h], rows),
                              1.0 / math.sqrt(128.0))
        hs = slice(h * G, (h + 1) * G)
        assert_attn_close(layer.out[0, 0, hs].cpu().numpy(), out, f"{cfg.name} head {h}")
        lse_close(layer.lse[0, 0, hs].cpu().numpy(), lse, f"{cfg.name} head {h}")

    # candidate mode on the same codes: the stored-score selection's indices
    want = layer.idx.clone()
    for flags in (0, sks.CAND_TEST_HIGH):
        flush(f"[max] candidate mode, flags {flags}")
        layer.score_candidates(flags=flags)
        layer.idx.fill_(-7)
        layer.select_candidates()
        torch.cuda.synchronize()
        assert torch.equal(layer.idx, want), flags


def test_most_segments():
    """8,191 sequences x 8 KV heads = 65,528 (sequence, KV head) segments, the
    most a grid dimension holds (65,535), on short rows: sampled segments
    (the first, the last and some between) against the oracle: sketches within
    the bound, scores and indices bit-exact given the GPU's codes, outputs
    within the output bound; the candidate mode's selection equal to the
    stored-score one on every segment."""
    B, HKV_, G_ = 8191, 8, 1
    cfg = C.Config("max_segments", 92, B=B, R=1, Hq=HKV_ * G_, Hkv=HKV_, L=64, window=16,
                   topk=8, pool=1, kv_dtype=C.KV_BF16, needle_kind="random", needle_count=2,
                   needle_amp=3.0, needle_noise=0.5)
    flush(f"[max] {B} x {HKV_} segments")
    case = make_case_on_device(cfg, "cuda")
    K, V = case.K, case.V
    sl = torch.from_numpy(case.seq_len.copy()).cuda()
    layer = SparseDecodeLayer(B, 1, HKV_ * G_, HKV_, cfg.T_max, 16, 8, 1, sks.KV_BF16)
    layer.bind(sks.Cache(K, V, sl), torch.from_numpy(case.basis).cuda(),
               torch.from_numpy(case.key_scale).cuda())
    q = torch.from_numpy(case.q.view(np.int16)).cuda().view(torch.bfloat16)
    layer.build_sketch(0, cfg.T_max)
    layer.step(q)
    torch.cuda.synchronize()
    n_far = cfg.L - 16
    qf = orc.bf16_to_f64(case.q)
    for b, h in [(0, 0), (B - 1, HKV_ - 1), (B // 2, 3), (1234, 5), (B - 2, 0)]:
        Kf = rows_f64(K[b, h], np.arange(cfg.L))
        Vf = rows_f64(V[b, h], np.arange(cfg.L))
        y = orc.project(Kf, case.basis)
        codes = layer.S[b, h].cpu().numpy()
        assert sketch_ok(codes[:cfg.L], y, float(case.key_scale[h])).all(), (b, h)
        qg = qf[b, 0, h * G_:(h + 1) * G_]
        _, qs, yq = orc.query_sketch(qg, case.basis)
        qc = layer.qsk[b, 0, h].cpu().numpy()
        assert sketch_ok(qc, yq, qs).all(), (b, h)
        sc = orc.scores(qc, codes[:n_far])
        assert np.array_equal(layer.scores[b, 0, h, :n_far].cpu().numpy().astype(np.int64), sc)
        sel = orc.select_topk(sc, 8)
        assert np.array_equal(layer.idx[b, 0, h].cpu().numpy(), sel.astype(np.int32)), (b, h)
        rows = np.concatenate([sel, np.arange(n_far, cfg.L)])
        out, lse = orc.attend(qg, Kf[rows], Vf[rows], 1.0 / math.sqrt(128.0))
        hs = slice(h * G_, (h + 1) * G_)
        assert_attn_close(layer.out[b, 0, hs].cpu().numpy(), out, f"{(b, h)}")
        lse_close(layer.lse[b, 0, hs].cpu().numpy(), lse, f"{(b, h)}")
    # candidate mode over all 65,528 segments: the stored-score selection
    want = layer.idx.clone()
    for flags in (0, sks.CAND_TEST_HIGH, sks.CAND_TEST_ZERO):
        layer.score_candidates(flags=flags)
        layer.idx.fill_(-7)
        layer.select_candidates()
        torch.cuda.synchronize()
        assert torch.equal(layer.idx, want), flags
