"""The step as sub-batches on several streams, and captured into a HIP graph
("CUDA-graph safe" in "What it took" of "8 agents x 250K context ... on two
3090s"): bit-identical to the single-stream eager step, on every replay, with
eager work and synchronisations between replays, and following device-side
lengths changed between replays."""
import numpy as np
import pytest
import torch

from long_context_sparse_sketch_amd import configs as C
from long_context_sparse_sketch_amd.runtime import StepRunner
from long_context_sparse_sketch_amd.synth import make_case
from tests.gpu_util import GpuCase, flush

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("cfg,parts,streams", [(C.small(C.C3), 2, 2), (C.small(C.C5), 2, 1),
                                               (C.small(C.C4), 2, 2),
                                               (C.with_kv(C.small(C.C5), C.KV_I4), 2, 1)],
                         ids=lambda x: str(x))
def test_streams_and_graph_replays_match_eager(cfg, parts, streams):
    flush(f"[graph] {cfg.name} parts={parts} streams={streams}")
    case = make_case(cfg)
    g = GpuCase(case)
    g.layer.build_sketch(0, g.T)
    g.layer.step(g.q)
    torch.cuda.synchronize()
    ref = [t.clone() for t in (g.layer.out, g.layer.lse, g.layer.idx)]

    runner = StepRunner(g.layer, parts=parts, streams=streams)
    g.layer.out.zero_(); g.layer.idx.zero_()
    runner.step(g.q)
    torch.cuda.synchronize()
    for a, b in zip(ref, (g.layer.out, g.layer.lse, g.layer.idx)):
        assert torch.equal(a, b)

    runner.capture(g.q)
    for rep in range(3):
        g.layer.out.zero_(); g.layer.lse.zero_(); g.layer.idx.fill_(-5)
        x = torch.randn(1000, device="cuda").sum()          # eager work between replays
        torch.cuda.synchronize()
        runner.replay()
        torch.cuda.synchronize()
        for a, b in zip(ref, (g.layer.out, g.layer.lse, g.layer.idx)):
            assert torch.equal(a, b), rep
        del x

    # the captured step reads lengths on the device
    g.seq_len.sub_(5)
    runner.replay()
    torch.cuda.synchronize()
    got = [t.clone() for t in (g.layer.out, g.layer.lse, g.layer.idx)]
    g.layer.step(g.q)
    torch.cuda.synchronize()
    for a, b in zip(got, (g.layer.out, g.layer.lse, g.layer.idx)):
        assert torch.equal(a, b)
    g.seq_len.add_(5)


@pytest.mark.parametrize("cfg", [C.small(C.C3), C.small(C.C4), C.with_kv(C.small(C.C5), C.KV_I4)],
                         ids=lambda c: c.name)
def test_candidate_selection_graph_replays(cfg):
    """The candidate mode's passes (sample, score, final) captured in a graph:
    every replay gives the stored-score selection's indices, with eager work
    between replays (its histograms return to zero each time), and the
    captured passes follow device-side lengths."""
    flush(f"[graph candidates] {cfg.name}")
    case = make_case(cfg)
    g = GpuCase(case)
    lay = g.layer
    lay.build_sketch(0, g.T)
    lay.step(g.q)
    torch.cuda.synchronize()
    want = lay.idx.clone()

    def sel():
        lay.score_candidates()
        lay.select_candidates()

    sel()                                                    # warm-up outside the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        sel()
    for rep in range(3):
        lay.idx.fill_(-5)
        x = torch.randn(1000, device="cuda").sum()          # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(lay.idx, want), rep
        del x
    g.seq_len.sub_(5)
    graph.replay()
    torch.cuda.synchronize()
    got = lay.idx.clone()
    lay.score()
    lay.select()
    torch.cuda.synchronize()
    assert torch.equal(got, lay.idx)
    g.seq_len.add_(5)
