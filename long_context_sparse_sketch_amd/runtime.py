"""Device buffers and call order of one sparse-sketch decode-attention layer.

`SparseDecodeLayer` owns the sketch cache, the per-step scratch (query
sketch, scores, indices, workspace) and the outputs for one shape, and issues
the C-ABI calls of a step on the current stream:

    sks_sketch_build(APPEND)      sketch of the rows' own (just appended) tokens
    sks_sketch_build_query        rank-64 int8 query sketch per KV head
    sks_sketch_score              int32 score of every far token / block, plus the
                                  selection's level-1 histogram in the workspace
    sks_topk_select               top-k indices, ascending, -1 padded
    sks_sparse_decode_attn        gather + one merged softmax over far + window

torch is used only to allocate device memory; no step calls back into it.
"""
from __future__ import annotations

import numpy as np
import torch

from . import binding as sks


def to_device(arr: np.ndarray, device="cuda", bf16=False) -> torch.Tensor:
    """Upload a numpy array; uint16 arrays holding bf16 bits become bfloat16."""
    a = np.ascontiguousarray(arr)
    if a.dtype == np.uint16:
        t = torch.from_numpy(a.view(np.int16))
        t = t.view(torch.bfloat16) if bf16 else t
    else:
        t = torch.from_numpy(a)
    return t.to(device)


def bits_u16(t: torch.Tensor) -> np.ndarray:
    """Host copy of a 16-bit tensor as raw uint16 bit patterns."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


class SparseDecodeLayer:
    def __init__(self, B, R, Hq, Hkv, T_max, window, topk, pool=1, kv_dtype=sks.KV_BF16,
                 device="cuda"):
        self.B, self.R, self.Hq, self.Hkv, self.T_max = B, R, Hq, Hkv, T_max
        self.window, self.topk, self.pool, self.kv_dtype = window, topk, pool, kv_dtype
        self.NB = T_max // pool
        self.p = sks.params(window, topk, pool, R)
        dev = device
        self.S = torch.empty((B, Hkv, self.NB, sks.RANK), dtype=torch.int8, device=dev)
        if pool > 1:
            self.Kp = torch.empty((B, Hkv, self.NB, sks.HEAD_DIM), dtype=torch.bfloat16, device=dev)
            self.Vp = torch.empty_like(self.Kp)
        else:
            self.Kp = self.Vp = None
        self.qsk = torch.empty((B, R, Hkv, sks.RANK), dtype=torch.int8, device=dev)
        self.qscale = torch.empty((B, R, Hkv), dtype=torch.float32, device=dev)
        self.scores = torch.empty((B, R, Hkv, self.NB), dtype=torch.int32, device=dev)
        self.idx = torch.empty((B, R, Hkv, topk), dtype=torch.int32, device=dev)
        self.n_sel = torch.empty((B, R, Hkv), dtype=torch.int32, device=dev)
        self.out = torch.empty((B, R, Hq, sks.HEAD_DIM), dtype=torch.float32, device=dev)
        self.lse = torch.empty((B, R, Hq), dtype=torch.float32, device=dev)
        self.cache = None
        self.ws = None

    def bind(self, cache: sks.Cache, basis: torch.Tensor, key_scale: torch.Tensor,
             basis_per_head=False):
        self.cache, self.basis, self.key_scale = cache, basis, key_scale
        self.basis_per_head = basis_per_head
        nbytes = sks.workspace_bytes(cache, self.p, self.Hq)
        if nbytes == 0:
            raise sks.SksError(sks.SKS_ERR_ARG, sks.last_error())
        self.ws = torch.empty((nbytes,), dtype=torch.uint8, device=cache.K.device)
        sks.workspace_init(self.ws)          # the histogram region is zero at rest
        return self

    # ---- individual calls
    def build_sketch(self, t_begin=0, t_end=None, stream=None):
        sks.sketch_build(self.cache, self.p, self.basis, self.key_scale, self.S, t_begin, t_end,
                         self.Kp, self.Vp, self.basis_per_head, stream)

    def query_sketch(self, q, stream=None):
        sks.sketch_build_query(q, self.Hkv, self.basis, self.qsk, self.qscale,
                               self.basis_per_head, stream)

    def score(self, stream=None, qsk=None, S=None, fuse_hist=True):
        """Scores; with fuse_hist the selection histogram is built in the same pass."""
        sks.sketch_score(self.qsk if qsk is None else qsk, self.S if S is None else S,
                         self.cache, self.p, self.scores, self.ws if fuse_hist else None, stream)

    def select(self, stream=None, scores=None, hist_ready=None):
        """Top-k; hist_ready defaults to True for the layer's own scores, which
        `score()` produced with the fused histogram."""
        if hist_ready is None:
            hist_ready = scores is None
        sks.topk_select(self.scores if scores is None else scores, self.cache, self.p, self.idx,
                        self.n_sel, self.ws, hist_ready, stream)

    def attend(self, q, stream=None, idx=None, sm_scale=None):
        sks.sparse_decode_attn(q, self.cache, self.p, self.idx if idx is None else idx, self.out,
                               self.ws, self.lse, self.Kp, self.Vp, sm_scale, stream)

    # ---- one decode step
    def step(self, q, stream=None, append=True):
        if append:
            self.build_sketch(sks.APPEND, 0, stream)
        self.query_sketch(q, stream)
        self.score(stream)
        self.select(stream)
        self.attend(q, stream)
        return self.out, self.lse
