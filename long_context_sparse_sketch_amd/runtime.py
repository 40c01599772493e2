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

or all of them as the one call sks_decode_step (the default of `step`).

torch is used only to allocate device memory and streams; no step calls back
into it.

`StepRunner` captures whole steps into HIP graphs (every call only enqueues
kernels and reads lengths on the device) and can schedule one step as
several sub-batches (views of the same buffers; segments never interact) on
a few streams, so that one part's latency-bound selection and attention
overlap another's score pass.  On the workloads measured here one stream is
the faster schedule: splitting pays every latency-bound kernel once per part.
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

    def view(self, b0: int, b1: int) -> "SparseDecodeLayer":
        """A layer over sequences [b0, b1) sharing this layer's buffers (own workspace)."""
        v = SparseDecodeLayer.__new__(SparseDecodeLayer)
        v.B, v.R, v.Hq, v.Hkv, v.T_max = b1 - b0, self.R, self.Hq, self.Hkv, self.T_max
        v.window, v.topk, v.pool, v.kv_dtype = self.window, self.topk, self.pool, self.kv_dtype
        v.NB, v.p = self.NB, self.p
        for name in ("S", "Kp", "Vp", "qsk", "qscale", "scores", "idx", "n_sel", "out", "lse"):
            t = getattr(self, name)
            setattr(v, name, None if t is None else t[b0:b1])
        c = self.cache
        sl = lambda t: None if t is None else t[b0:b1]
        cache = sks.Cache(c.K[b0:b1], c.V[b0:b1], c.seq_len[b0:b1], sl(c.K_scale), sl(c.V_scale),
                          None if c.hot is None else tuple(sl(t) for t in c.hot))
        v.cache, v.ws = None, None
        v.bind(cache, self.basis, self.key_scale, self.basis_per_head)
        return v

    def bind(self, cache: sks.Cache, basis: torch.Tensor, key_scale: torch.Tensor,
             basis_per_head=False):
        self.cache, self.basis, self.key_scale = cache, basis, key_scale
        self.basis_per_head = basis_per_head
        nbytes = sks.workspace_bytes(cache, self.p, self.Hq)
        if nbytes == 0:
            raise sks.SksError(sks.SKS_ERR_ARG, sks.last_error())
        self.ws = torch.empty((nbytes,), dtype=torch.uint8, device=cache.seq_len.device)
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

    def score_candidates(self, stream=None, qsk=None, S=None, flags=0):
        """Candidate mode's score pass: no scores stored (see select_candidates)."""
        sks.score_candidates(self.qsk if qsk is None else qsk, self.S if S is None else S,
                             self.cache, self.p, self.ws, flags, stream)

    def select_candidates(self, stream=None, qsk=None, S=None):
        """Selection from score_candidates' lists (self.scores is scratch)."""
        sks.topk_select_candidates(self.qsk if qsk is None else qsk, self.S if S is None else S,
                                   self.cache, self.p, self.scores, self.idx, self.n_sel,
                                   self.ws, stream)

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
    def dense_covers(self, max_len: int) -> bool:
        """True when a dense step attends exactly the sparse step's set for
        rows up to max_len tokens (the switch: dense for short rows)."""
        return self.pool == 1 and max_len + self.R - 1 <= self.window + self.topk

    def step(self, q, stream=None, append=True, fused=True, dense=False, keep_scores=True):
        """One step; `fused` issues it as the single sks_decode_step call,
        otherwise as the individual calls (same results).  `dense` skips
        scoring and selection (one call only).  keep_scores=False lets the
        fused step run the selection in candidate mode, which stores no
        scores (same idx, out and lse)."""
        if fused or dense:
            sks.decode_step(self.cache, self.p, q, self.basis, self.key_scale, self.S, self.qsk,
                            self.scores, self.idx, self.out, self.ws, qscale=self.qscale,
                            n_sel=self.n_sel, lse=self.lse, Kp=self.Kp, Vp=self.Vp,
                            basis_per_head=self.basis_per_head, append=append, dense=dense,
                            keep_scores=keep_scores, stream=stream)
            return self.out, self.lse
        if append:
            self.build_sketch(sks.APPEND, 0, stream)
        self.query_sketch(q, stream)
        self.score(stream)
        self.select(stream)
        self.attend(q, stream)
        return self.out, self.lse


class StepRunner:
    """One decode step of a layer, split into `parts` sub-batches on `streams`
    streams (fork/join on the caller's current stream), optionally captured
    into a HIP graph and replayed.  `dense`: the step without selection (the
    caller's switch for short rows, see SparseDecodeLayer.dense_covers).
    `keep_scores=False`: the scores buffer is scratch (candidate mode)."""

    def __init__(self, layer: SparseDecodeLayer, parts: int = 1, streams: int = 1,
                 overlap_append: bool = False, fused: bool = True, dense: bool = False,
                 keep_scores: bool = True):
        parts = max(1, min(parts, layer.B))
        bounds = [layer.B * k // parts for k in range(parts + 1)]
        self.layer = layer
        self.views = [layer.view(bounds[k], bounds[k + 1]) for k in range(parts)]
        self.bounds = bounds
        dev = layer.S.device
        self.streams = [torch.cuda.Stream(device=dev) for _ in range(max(1, streams))]
        self.append_stream = torch.cuda.Stream(device=dev) if overlap_append else None
        self.graph = None
        self.fused = fused
        self.dense = dense
        self.keep_scores = keep_scores

    def step(self, q):
        main = torch.cuda.current_stream()
        for st in self.streams:
            st.wait_stream(main)
        # The rows' own tokens lie inside every row's exact window when
        # window >= rows, so this step's scoring never reads the sketches the
        # append writes: the append then runs beside the query/score chain.
        side = self.append_stream if self.layer.window >= self.layer.R else None
        if side is None and len(self.streams) == 1 and len(self.views) == 1:
            # plain single-stream step on the caller's stream
            self.views[0].step(q, fused=self.fused, dense=self.dense,
                               keep_scores=self.keep_scores)
            return self.layer.out, self.layer.lse
        if side is not None:
            side.wait_stream(main)
            with torch.cuda.stream(side):
                for v in self.views:
                    v.build_sketch(sks.APPEND, 0)
        for k, v in enumerate(self.views):
            st = self.streams[k % len(self.streams)]
            with torch.cuda.stream(st):
                v.step(q[self.bounds[k]:self.bounds[k + 1]], append=side is None, fused=self.fused,
                       dense=self.dense, keep_scores=self.keep_scores)
        for st in self.streams:
            main.wait_stream(st)
        if side is not None:
            main.wait_stream(side)
        return self.layer.out, self.layer.lse

    def capture(self, q):
        """Capture step(q) (q: a static input tensor) into a graph."""
        self.graph = capture_steps([self], q)
        return self.graph

    def replay(self):
        self.graph.replay()
        return self.layer.out, self.layer.lse


def capture_steps(runners, q):
    """Capture one step of each runner, in order, into ONE HIP graph (e.g. the
    layers of a decode iteration), so that a single launch replays them all."""
    for r in runners:                                  # warm up outside the capture
        r.step(q)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for r in runners:
            r.step(q)
    torch.cuda.synchronize()
    return g
