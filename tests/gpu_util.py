"""Helpers shared by the GPU parity tests: upload a synthetic case, run the
HIP path through the C ABI, run the oracle, and compare to the stated bars.

Bars (from the method's acceptance rules):
* sketch codes: |s * code_gpu - clamp(y)| <= s/2 + 1e-2 |y| elementwise, with
  y the oracle's float64 projection and s the scale (a code may only differ
  where y/s sits next to a rounding boundary);
* scores and indices: bit-exact when both sides are fed the same int8 sketches;
* attention: |o_gpu - o_ref| <= 1e-3 + 2e-3 |o_ref| against the float64 oracle.
"""
from __future__ import annotations

import math

import numpy as np
import torch

from long_context_sparse_sketch_amd import binding as sks
from long_context_sparse_sketch_amd import configs as C
from long_context_sparse_sketch_amd.runtime import SparseDecodeLayer, bits_u16, to_device
from oracle import sks_oracle as orc

RTOL, ATOL = 2e-3, 1e-3


def flush(msg: str):
    print(msg, flush=True)


class GpuCase:
    """A synthetic case resident on the GPU with its layer buffers."""

    def __init__(self, case, seq_len=None, topk=None, window=None, pool=None):
        cfg = case.cfg
        self.case, self.cfg = case, cfg
        self.topk = cfg.topk if topk is None else topk
        self.window = cfg.window if window is None else window
        self.pool = cfg.pool if pool is None else pool
        B = case.B
        T = case.K.shape[2]
        self.T = T
        codes = cfg.kv_dtype != C.KV_BF16      # int8 codes, or packed int4 bytes
        self.K = to_device(case.K, bf16=True) if not codes else torch.from_numpy(case.K).cuda()
        self.V = to_device(case.V, bf16=True) if not codes else torch.from_numpy(case.V).cuda()
        self.Ks = to_device(case.K_scale) if codes else None
        self.Vs = to_device(case.V_scale) if codes else None
        sl = case.seq_len if seq_len is None else np.asarray(seq_len, np.int32)
        self.seq_len_np = sl
        self.seq_len = torch.from_numpy(sl.copy()).cuda()
        self.q = to_device(case.q, bf16=True)
        self.basis = torch.from_numpy(case.basis).cuda()
        self.key_scale = torch.from_numpy(case.key_scale).cuda()
        self.cache = sks.Cache(self.K, self.V, self.seq_len, self.Ks, self.Vs)
        self.layer = SparseDecodeLayer(B, cfg.R, cfg.Hq, cfg.Hkv, T, self.window, self.topk,
                                       self.pool, cfg.kv_dtype).bind(self.cache, self.basis,
                                                                      self.key_scale)

    def run_full(self):
        self.layer.build_sketch(0, self.T)
        out, lse = self.layer.step(self.q)
        torch.cuda.synchronize()
        return out, lse

    def oracle(self, heads=None, codes=None):
        """The oracle's step on this case; `codes` = (key codes [B][Hkv][NB][64],
        query codes [B][R][Hkv][64]) makes it score, select and attend from
        those int8 sketches (e.g. the GPU's own) instead of its own."""
        c, cfg = self.case, self.cfg
        return orc.decode_step(c.q, c.K, c.V, c.K_scale, c.V_scale, self.seq_len_np, c.basis,
                               c.key_scale, self.window, self.topk, self.pool,
                               cfg.kv_dtype, heads=heads, codes=codes)


def sketch_ok(code_gpu: np.ndarray, y: np.ndarray, s: float):
    """Elementwise sketch acceptance; returns (ok_mask, n_code_mismatch)."""
    lim = 127.0 * s
    yc = np.clip(y, -lim, lim)
    ok = np.abs(s * code_gpu.astype(np.float64) - yc) <= s / 2 + 1e-2 * np.abs(y)
    return ok


def oracle_key_projection(case, b, h, pool):
    """Float64 projection y of every sketch row of (b, h), from the oracle."""
    cfg = case.cfg
    Kf, Vf = orc.cache_rows(case.K, case.V, case.K_scale, case.V_scale, b, h,
                            cfg.kv_dtype)
    Kp = orc.pool_mean(Kf, pool)
    return orc.project(Kp, case.basis), Kp, orc.pool_mean(Vf, pool)


def assert_attn_close(out_gpu, out_ref, what=""):
    np.testing.assert_allclose(out_gpu, out_ref, rtol=RTOL, atol=ATOL, err_msg=what)


def lse_close(lse_gpu, lse_ref, what=""):
    finite = np.isfinite(lse_ref)
    assert np.array_equal(np.isfinite(lse_gpu), finite), what
    np.testing.assert_allclose(lse_gpu[finite], lse_ref[finite], rtol=RTOL, atol=ATOL, err_msg=what)


def ref_arrays(ref, cfg, B, topk, NB):
    """Stack oracle per-(b,h) results into the GPU layouts."""
    R, Hkv, g = cfg.R, cfg.Hkv, cfg.g
    idx = np.full((B, R, Hkv, topk), -1, np.int32)
    n_sel = np.zeros((B, R, Hkv), np.int32)
    out = np.zeros((B, R, cfg.Hq, 128))
    lse = np.zeros((B, R, cfg.Hq))
    scores = np.zeros((B, R, Hkv, NB), np.int64)
    kcodes = np.zeros((B, Hkv, NB, 64), np.int8)
    qcode = np.zeros((B, R, Hkv, 64), np.int8)
    qscale = np.zeros((B, R, Hkv))
    for (b, h), r in ref.items():
        kcodes[b, h] = r["kcodes"][:NB]
        for i in range(R):
            idx[b, i, h] = r["idx"][i]
            n_sel[b, i, h] = r["n_sel"][i]
            out[b, i, h * g:(h + 1) * g] = r["out"][i]
            lse[b, i, h * g:(h + 1) * g] = r["lse"][i]
            scores[b, i, h, :len(r["scores"][i])] = r["scores"][i]
            qcode[b, i, h] = r["qcode"][i]
            qscale[b, i, h] = r["qscale"][i]
    return dict(idx=idx, n_sel=n_sel, out=out, lse=lse, scores=scores, kcodes=kcodes,
                qcode=qcode, qscale=qscale)


def sm_default():
    return 1.0 / math.sqrt(128.0)


__all__ = ["GpuCase", "sketch_ok", "oracle_key_projection", "assert_attn_close", "lse_close",
           "ref_arrays", "bits_u16", "flush", "RTOL", "ATOL"]


def run_arrays(q, K, V, seq_len, basis, key_scale, window, topk, pool=1, Ks=None, Vs=None,
               ref=None, basis_per_head=False):
    """Run one full GPU step (bulk sketch + step) on raw host arrays.

    q: [B][R][Hq][128] bf16 bits; K, V: [B][Hkv][T][128] bf16 bits or int8.
    With `ref` (an oracle result for every (b, h)), the scoring, selection and
    attention run on the oracle's int8 key and query codes instead of the
    GPU's, so that indices can be compared bit for bit.
    Returns numpy copies of every intermediate and output.
    """
    from long_context_sparse_sketch_amd.runtime import SparseDecodeLayer
    B, R, Hq, _ = q.shape
    Hkv, T = K.shape[1], K.shape[2]
    i8 = K.dtype == np.int8
    Kd = torch.from_numpy(K).cuda() if i8 else to_device(K, bf16=True)
    Vd = torch.from_numpy(V).cuda() if i8 else to_device(V, bf16=True)
    Ksd = to_device(Ks) if i8 else None
    Vsd = to_device(Vs) if i8 else None
    sl = torch.from_numpy(np.asarray(seq_len, np.int32).copy()).cuda()
    cache = sks.Cache(Kd, Vd, sl, Ksd, Vsd)
    layer = SparseDecodeLayer(B, R, Hq, Hkv, T, window, topk, pool,
                              sks.KV_I8 if i8 else sks.KV_BF16)
    layer.bind(cache, torch.from_numpy(np.ascontiguousarray(basis, np.float32)).cuda(),
               torch.from_numpy(np.ascontiguousarray(key_scale, np.float32)).cuda(),
               basis_per_head=basis_per_head)
    layer.build_sketch(0, T)
    qd = to_device(q, bf16=True)
    if ref is None:
        layer.step(qd)
    else:
        layer.query_sketch(qd)
        kc = np.zeros((B, Hkv, layer.NB, 64), np.int8)
        qc = np.zeros((B, R, Hkv, 64), np.int8)
        for (b, h), o in ref.items():
            kc[b, h] = o["kcodes"][:layer.NB]
            for i in range(R):
                qc[b, i, h] = o["qcode"][i]
        layer.score(qsk=torch.from_numpy(qc).cuda(), S=torch.from_numpy(kc).cuda())
        layer.select()
        layer.attend(qd)
    torch.cuda.synchronize()
    return dict(S=layer.S.cpu().numpy(), qsk=layer.qsk.cpu().numpy(),
                scores=layer.scores.cpu().numpy(), idx=layer.idx.cpu().numpy(),
                n_sel=layer.n_sel.cpu().numpy(), out=layer.out.cpu().numpy(),
                lse=layer.lse.cpu().numpy(), layer=layer, cache=cache)
