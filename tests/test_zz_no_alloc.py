"""The allocation-free step (sks_decode_step_static, through the C ABI)
against sks_decode_step with a caller-provided workspace: the same bits in
every output buffer, on consecutive calls of different shapes on one GPU (the
second smaller than the first, then the first again), so that each call finds
the previous call's contents in the shared static workspace."""
import numpy as np
import pytest
import torch

from long_context_sparse_sketch_amd import binding as sks
from long_context_sparse_sketch_amd import configs as C
from long_context_sparse_sketch_amd.synth import make_case
from tests.gpu_util import GpuCase, flush

pytestmark = pytest.mark.gpu

OUTS = ("S", "qsk", "qscale", "scores", "idx", "n_sel", "out", "lse")


def run(g, static, keep_scores):
    lay = g.layer
    for n in OUTS[1:]:
        getattr(lay, n).view(torch.uint8).fill_(0x5A)
    lay.build_sketch(0, g.T)                  # the same sketch before each step
    kw = dict(qscale=lay.qscale, n_sel=lay.n_sel, lse=lay.lse, Kp=lay.Kp, Vp=lay.Vp,
              basis_per_head=lay.basis_per_head, keep_scores=keep_scores)
    if static:
        sks.decode_step_static(lay.cache, lay.p, g.q, lay.basis, lay.key_scale, lay.S, lay.qsk,
                               lay.scores, lay.idx, lay.out, **kw)
    else:
        sks.decode_step(lay.cache, lay.p, g.q, lay.basis, lay.key_scale, lay.S, lay.qsk,
                        lay.scores, lay.idx, lay.out, lay.ws, **kw)
    torch.cuda.synchronize()
    names = OUTS if keep_scores else tuple(n for n in OUTS if n != "scores")
    if lay.Kp is not None:
        names += ("Kp", "Vp")
    return {n: getattr(lay, n).clone() for n in names}


# first a long batch (the selection in candidate mode), then a smaller shape
# with verify rows and an int8 cache, then a pooled one, then the first again
SHAPES = [
    (C.C3.scaled(name="cand_8x40000", B=8, L=40000), False),
    (C.small(C.C5), True),
    (C.small(C.C4), True),
    (C.C3.scaled(name="cand_8x40000", B=8, L=40000), False),
]


def test_static_step_equals_workspace_step_on_consecutive_shapes():
    assert SHAPES[1][0].B * SHAPES[1][0].L < SHAPES[0][0].B * SHAPES[0][0].L
    cases = {}
    for cfg, keep in SHAPES:
        flush(f"[no-alloc] {cfg.name} keep_scores={keep}")
        if cfg.name not in cases:
            cases[cfg.name] = GpuCase(make_case(cfg))
        g = cases[cfg.name]
        want = run(g, static=False, keep_scores=keep)
        for _ in range(2):                    # the same shape twice in a row as well
            got = run(g, static=True, keep_scores=keep)
            for n in want:
                assert torch.equal(want[n].view(torch.uint8), got[n].view(torch.uint8)), \
                    (cfg.name, n)

