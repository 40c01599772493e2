"""The dense half of the per-step dense/sparse switch ("8 agents x 250K
context ...", "What it took": switch dense/sparse per step so that short
chats stay at full speed): sks_decode_step with SKS_STEP_DENSE skips scoring
and selection and attends each row's last window + topk tokens.

Checked against the oracle run with that window and no selection, for rows
shorter and longer than window + topk; for short unpooled rows also against
the sparse step (the same attention set, so the same outputs up to rounding),
and the APPEND sketch rows against the sparse step's, bit for bit."""
import numpy as np
import pytest
import torch

from long_context_sparse_sketch_amd import configs as C
from long_context_sparse_sketch_amd.runtime import StepRunner
from long_context_sparse_sketch_amd.synth import make_case
from oracle import sks_oracle as orc
from tests.gpu_util import GpuCase, assert_attn_close, flush, lse_close, ref_arrays

pytestmark = pytest.mark.gpu

CASES = [
    (C.small(C.C3), True), (C.small(C.C3), False),
    (C.small(C.C5), True), (C.small(C.C5), False),
    (C.with_kv(C.small(C.C5), C.KV_I4), True),
    (C.small(C.C4), False),
    (C.C1, True),
]


def lengths(cfg, B, short):
    if short:   # every row within window + topk, the last row of sequence 0 at the bound
        top = cfg.window + cfg.topk - (cfg.R - 1)
        return np.array([top - 997 * b for b in range(B)], np.int32)
    return np.array([cfg.L - 13 * b for b in range(B)], np.int32)


@pytest.mark.parametrize("cfg,short", CASES,
                         ids=[c.name + ("_short" if s else "_long") for c, s in CASES])
def test_dense_step(cfg, short):
    case = make_case(cfg)
    sl = lengths(cfg, case.B, short)
    flush(f"[dense] {cfg.name}: lengths {sl.tolist()}")
    g = GpuCase(case, seq_len=sl)
    g.layer.build_sketch(0, g.T)
    S0 = g.layer.S.clone()
    g.layer.step(g.q, dense=True)
    torch.cuda.synchronize()
    out_d, lse_d = g.layer.out.cpu().numpy(), g.layer.lse.cpu().numpy()
    S_d = g.layer.S.clone()

    c = case
    ref = orc.decode_step(c.q, c.K, c.V, c.K_scale, c.V_scale, sl, c.basis, c.key_scale,
                          g.window + g.topk, 0, g.pool, cfg.kv_dtype)
    arr = ref_arrays(ref, cfg, case.B, 0, g.layer.NB)
    assert_attn_close(out_d, arr["out"], cfg.name)
    lse_close(lse_d, arr["lse"], cfg.name)

    # the sparse step: the same APPEND rows; for short unpooled rows the same set
    g.layer.S.copy_(S0)
    g.layer.step(g.q)
    torch.cuda.synchronize()
    assert torch.equal(S_d, g.layer.S)
    if short and cfg.pool == 1:
        assert g.layer.dense_covers(int(sl.max()))
        assert_attn_close(out_d, g.layer.out.cpu().numpy(), cfg.name + " vs sparse")
        lse_close(lse_d, g.layer.lse.cpu().numpy(), cfg.name + " vs sparse")


def test_dense_step_graph_replays():
    cfg = C.small(C.C3)
    case = make_case(cfg)
    g = GpuCase(case)
    g.layer.build_sketch(0, g.T)
    g.layer.step(g.q, dense=True)
    torch.cuda.synchronize()
    want = (g.layer.out.clone(), g.layer.lse.clone())
    runner = StepRunner(g.layer, dense=True)
    runner.capture(g.q)
    for rep in range(3):
        g.layer.out.zero_()
        g.layer.lse.zero_()
        torch.cuda.synchronize()
        runner.replay()
        torch.cuda.synchronize()
        assert torch.equal(g.layer.out, want[0]) and torch.equal(g.layer.lse, want[1]), rep


def test_dense_step_full_size_graph():
    """The 8 x 250K benchmark cache through a graph-replayed dense step (as
    bench.py --dense times it): sampled (sequence, KV head) pairs against the
    oracle over each row's last window + topk tokens."""
    cfg = C.C3
    flush(f"[dense] full size {cfg.name}")
    case = make_case(cfg)
    g = GpuCase(case)
    g.layer.build_sketch(0, g.T)
    runner = StepRunner(g.layer, dense=True)
    runner.capture(g.q)
    runner.replay()
    torch.cuda.synchronize()
    pairs = sorted({(0, 0), (cfg.B - 1, cfg.Hkv - 1), (cfg.B // 2, cfg.Hkv // 2)})
    c = case
    ref = orc.decode_step(c.q, c.K, c.V, None, None, c.seq_len, c.basis, c.key_scale,
                          g.window + g.topk, 0, 1, cfg.kv_dtype, heads=pairs)
    out, lse = g.layer.out.cpu().numpy(), g.layer.lse.cpu().numpy()
    for (b, h), r in ref.items():
        sl = slice(h * cfg.g, (h + 1) * cfg.g)
        assert_attn_close(out[b, 0, sl], r["out"][0], f"{(b, h)}")
        lse_close(lse[b, 0, sl], r["lse"][0], f"{(b, h)}")
