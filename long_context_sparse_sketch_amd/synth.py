"""Seeded synthetic inputs for the sparse-sketch decode path.

This module only draws inputs; it performs none of the method's arithmetic
(no sketching, scoring, selection, pooling or attention).  Both the HIP path
(through tests and the benchmark) and the CPU oracle are fed from here.

Recipe (stand-ins for the pages' workloads, which used real model caches and
retrieval evals that are not available):

* basis: QR of a 128x64 N(0,1) float64 matrix; the orthonormal columns are
  stored as rows of a float32 ``[64][128]`` array (one frozen basis shared by
  all KV heads, as the "A frozen sketch basis (one file)" item of the
  "What it took" list of "8 agents x 250K context ... on two 3090s" suggests).
* q, K, V: float32 N(0,1) rounded to bfloat16 (round to nearest even).  For the
  int8 cache, each (token, KV head) row of K and of V gets
  ``scale = fp16(absmax / 127)`` and ``code = clip(rint(x / scale), -127, 127)``;
  the int4 cache likewise with 7 in place of 127, two codes per byte (dimension
  2j in the low nibble of byte j, 2j+1 in the high nibble, two's complement).
* needles: keys planted as ``amp * qbar_h + N(0, noise^2)`` where ``qbar_h`` is
  the mean of KV head h's group of (bf16) query vectors of row 0.  Kinds:
  ``random`` (count per KV head, uniform positions without replacement in the
  prior context), ``clusters`` (count per sequence, in 8 contiguous runs shared
  by all KV heads), ``blocks`` (count whole pool-aligned blocks per KV head in
  the far field), ``row0`` (as ``random``, aimed at row 0 of a verify step).

Every array of sequence b is drawn from streams keyed by (seed, tag, b, ...),
so a sequence's data does not depend on the batch it is generated in.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

from .configs import Config, KV_BF16, KV_I4, KV_I8

_TAG_BASIS, _TAG_Q, _TAG_K, _TAG_V, _TAG_POS, _TAG_NOISE = range(6)


def _rng(seed: int, *key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=key)))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Encode float32 as bfloat16 bit patterns, rounding to nearest even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u >> 16) & 1
    return ((u + 0x7FFF + r) >> 16).astype(np.uint16)


def _bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)


def _quantize_rows(x: np.ndarray, cmax: int):
    amax = np.abs(x).max(axis=-1)
    scale16 = (amax / np.float32(cmax)).astype(np.float16)
    s = scale16.astype(np.float32)
    safe = np.where(s > 0, s, np.float32(1.0))
    codes = np.clip(np.rint(x / safe[..., None]), -cmax, cmax)
    codes = np.where(s[..., None] > 0, codes, 0).astype(np.int8)
    return codes, scale16.view(np.uint16)


def quantize_rows_i8(x: np.ndarray):
    """Per-row symmetric int8 with an fp16 scale (the int8 cache encoding)."""
    return _quantize_rows(x, 127)


def pack_i4(codes: np.ndarray) -> np.ndarray:
    """int4 codes [..][128] in [-8, 7] -> bytes [..][64]: dimension 2j in the
    low nibble of byte j, dimension 2j+1 in the high nibble."""
    c = np.asarray(codes, dtype=np.int64)
    if c.size and (c.min() < -8 or c.max() > 7):
        raise ValueError("int4 codes must lie in [-8, 7]")
    u = (c & 0xF).astype(np.uint8)
    return (u[..., 0::2] | (u[..., 1::2] << 4)).astype(np.uint8)


def quantize_rows_i4(x: np.ndarray):
    """Per-row symmetric int4 (codes in [-7, 7]) with an fp16 scale, packed."""
    codes, scale = _quantize_rows(x, 7)
    return pack_i4(codes), scale


@dataclass
class Case:
    cfg: Config
    seqs: tuple                 # which sequence ids of the config these rows are
    basis: np.ndarray           # [64][128] float32
    key_scale: np.ndarray       # [Hkv] float32
    q: np.ndarray               # [B][R][Hq][128] uint16 (bf16 bits)
    K: np.ndarray               # [B][Hkv][T][128] uint16 (bf16) or int8; [..][64] uint8 (int4)
    V: np.ndarray
    K_scale: np.ndarray | None  # [B][Hkv][T] uint16 (fp16 bits) for int8 / int4
    V_scale: np.ndarray | None
    seq_len: np.ndarray         # [B] int32, length of row 0
    needles: dict = field(default_factory=dict)   # (b, h) -> sorted token positions

    @property
    def B(self) -> int:
        return self.q.shape[0]


def make_basis(cfg: Config) -> np.ndarray:
    g = _rng(cfg.seed, _TAG_BASIS)
    a = g.standard_normal((cfg.D, cfg.rank))
    qm, _ = np.linalg.qr(a)
    return np.ascontiguousarray(qm.T.astype(np.float32))


def _query(cfg: Config, b: int) -> np.ndarray:
    g = _rng(cfg.seed, _TAG_Q, b)
    return f32_to_bf16_bits(g.standard_normal((cfg.R, cfg.Hq, cfg.D), dtype=np.float32))


def _cluster_positions(cfg: Config, b: int, L_ctx: int) -> np.ndarray:
    n = min(cfg.needle_count, L_ctx)
    nclu = 8
    sizes = [n // nclu + (1 if i < n % nclu else 0) for i in range(nclu)]
    g = _rng(cfg.seed, _TAG_POS, b)
    offs = np.sort(g.integers(0, L_ctx - n + 1, size=nclu))
    pos, acc = [], 0
    for o, s in zip(offs, sizes):
        pos.append(np.arange(o + acc, o + acc + s))
        acc += s
    return np.concatenate(pos).astype(np.int64)


def _needle_positions(cfg: Config, b: int, h: int, L_ctx: int) -> np.ndarray:
    kind = cfg.needle_kind
    if kind == "clusters":
        return _cluster_positions(cfg, b, L_ctx)
    g = _rng(cfg.seed, _TAG_POS, b, h)
    if kind in ("random", "row0"):
        n = min(cfg.needle_count, L_ctx)
        return np.sort(g.choice(L_ctx, size=n, replace=False)).astype(np.int64)
    if kind == "blocks":
        r = cfg.pool
        nblk = cfg.n_far(0)
        n = min(cfg.needle_count, nblk)
        blk = np.sort(g.choice(nblk, size=n, replace=False))
        return (blk[:, None] * r + np.arange(r)[None, :]).reshape(-1).astype(np.int64)
    raise ValueError(kind)


def _kv_block(cfg: Config, b: int, h: int, qbar: np.ndarray):
    T = cfg.T_max
    gk = _rng(cfg.seed, _TAG_K, b, h)
    gv = _rng(cfg.seed, _TAG_V, b, h)
    k = gk.standard_normal((T, cfg.D), dtype=np.float32)
    v = gv.standard_normal((T, cfg.D), dtype=np.float32)
    # needles live in the prior context: not on the query rows' own tokens
    pos = _needle_positions(cfg, b, h, cfg.L - 1)
    if pos.size:
        gn = _rng(cfg.seed, _TAG_NOISE, b, h)
        noise = gn.standard_normal((pos.size, cfg.D), dtype=np.float32) * np.float32(cfg.needle_noise)
        k[pos] = np.float32(cfg.needle_amp) * qbar[None, :] + noise
    if cfg.kv_dtype == KV_BF16:
        return f32_to_bf16_bits(k), f32_to_bf16_bits(v), None, None, pos
    quant = quantize_rows_i8 if cfg.kv_dtype == KV_I8 else quantize_rows_i4
    kc, ks = quant(k)
    vc, vs = quant(v)
    return kc, vc, ks, vs, pos


def make_case(cfg: Config, seqs=None, threads: int | None = None) -> Case:
    """Draw the inputs of `cfg` for the sequences `seqs` (default: all)."""
    seqs = tuple(range(cfg.B)) if seqs is None else tuple(seqs)
    B, T = len(seqs), cfg.T_max
    basis = make_basis(cfg)
    key_scale = np.full((cfg.Hkv,), 1.0 / 16.0, dtype=np.float32)
    q = np.stack([_query(cfg, b) for b in seqs]) if B else np.zeros((0, cfg.R, cfg.Hq, cfg.D), np.uint16)
    kv_np = {KV_BF16: np.uint16, KV_I8: np.int8, KV_I4: np.uint8}[cfg.kv_dtype]
    row = cfg.D // 2 if cfg.kv_dtype == KV_I4 else cfg.D
    K = np.empty((B, cfg.Hkv, T, row), dtype=kv_np)
    V = np.empty_like(K)
    Ks = Vs = None
    if cfg.kv_dtype != KV_BF16:
        Ks = np.empty((B, cfg.Hkv, T), dtype=np.uint16)
        Vs = np.empty_like(Ks)
    qf = _bf16_bits_to_f32(q) if B else None
    needles = {}

    def work(item):
        bi, h = item
        qbar = qf[bi, 0, h * cfg.g:(h + 1) * cfg.g].astype(np.float64).mean(axis=0).astype(np.float32)
        kk, vv, ks, vs, pos = _kv_block(cfg, seqs[bi], h, qbar)
        K[bi, h] = kk
        V[bi, h] = vv
        if Ks is not None:
            Ks[bi, h] = ks
            Vs[bi, h] = vs
        needles[(bi, h)] = pos

    items = [(bi, h) for bi in range(B) for h in range(cfg.Hkv)]
    nthr = threads or min(16, os.cpu_count() or 1)
    if nthr > 1 and len(items) > 1:
        with ThreadPoolExecutor(nthr) as ex:
            list(ex.map(work, items))
    else:
        for it in items:
            work(it)
    seq_len = np.full((B,), cfg.L, dtype=np.int32)
    return Case(cfg, seqs, basis, key_scale, q, K, V, Ks, Vs, seq_len, needles)


def random_arrays(B: int, R: int, Hq: int, Hkv: int, T: int, seed: int, i8: bool = False):
    """Plain random inputs for edge-case tests, from one seeded stream:
    q [B][R][Hq][128] bf16 bits, K, V [B][Hkv][T][128] (bf16 bits, or int8
    codes with fp16 row scales Ks, Vs), a QR basis [64][128] and key scales
    of 1/16.  Returns (q, K, V, Ks, Vs, basis, key_scale)."""
    rng = np.random.default_rng(seed)
    q = f32_to_bf16_bits(rng.standard_normal((B, R, Hq, 128)).astype(np.float32))
    basis = np.linalg.qr(rng.standard_normal((128, 64)))[0].T.astype(np.float32)
    ks = np.full(Hkv, 1 / 16, np.float32)
    if not i8:
        K = f32_to_bf16_bits(rng.standard_normal((B, Hkv, T, 128)).astype(np.float32))
        V = f32_to_bf16_bits(rng.standard_normal((B, Hkv, T, 128)).astype(np.float32))
        return q, K, V, None, None, basis, ks
    K, Ks = quantize_rows_i8(rng.standard_normal((B, Hkv, T, 128)).astype(np.float32))
    V, Vs = quantize_rows_i8(rng.standard_normal((B, Hkv, T, 128)).astype(np.float32))
    return q, K, V, Ks, Vs, basis, ks


def random_scores(shape, lo: int, hi: int, seed: int) -> np.ndarray:
    """int32 scores drawn uniformly from [lo, hi] (narrow ranges: dense ties)."""
    return np.random.default_rng(seed).integers(lo, hi + 1, shape).astype(np.int32)


def distinct_diagonal(n: int, seed: int) -> np.ndarray:
    """The values 1..n in a seeded random order (a diagonal with distinct entries)."""
    return np.random.default_rng(seed).permutation(n).astype(np.float64) + 1.0


_TAG_DEVICE = 101


def make_case_on_device(cfg: Config, device) -> Case:
    """The inputs of a bf16-cache `cfg` with K and V drawn on `device`, for
    caches too large to draw on the host in reasonable time (millions of
    tokens per sequence): K, V are N(0,1) from torch's generator on the
    device, seeded from (seed, tag), rounded to bf16 by torch (nearest even);
    q, basis, key scale, needle positions and needle rows as in `make_case`.
    Returns a Case whose K and V are device tensors [B][Hkv][T][128] bf16."""
    import torch

    if cfg.kv_dtype != KV_BF16:
        raise ValueError("make_case_on_device draws bf16 caches only")
    B, T, D = cfg.B, cfg.T_max, cfg.D
    basis = make_basis(cfg)
    key_scale = np.full((cfg.Hkv,), 1.0 / 16.0, dtype=np.float32)
    q = np.stack([_query(cfg, b) for b in range(B)])
    qf = _bf16_bits_to_f32(q)
    seed = int(np.random.SeedSequence(cfg.seed, spawn_key=(_TAG_DEVICE,)).generate_state(1)[0])
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    K = torch.empty((B, cfg.Hkv, T, D), dtype=torch.bfloat16, device=device)
    V = torch.empty_like(K)
    # K, then V, over the flattened cache in chunks of 4M rows
    chunk = 1 << 22
    n = B * cfg.Hkv * T
    for dst in (K.view(n, D), V.view(n, D)):
        for r0 in range(0, n, chunk):
            r1 = min(n, r0 + chunk)
            dst[r0:r1] = torch.randn((r1 - r0, D), generator=gen, device=device,
                                     dtype=torch.float32).to(torch.bfloat16)
    # needles: every (sequence, KV head)'s rows planted with one indexed write
    needles, at, rows = {}, [], []
    for b in range(B):
        for h in range(cfg.Hkv):
            pos = _needle_positions(cfg, b, h, cfg.L - 1)
            needles[(b, h)] = pos
            if pos.size:
                qbar = qf[b, 0, h * cfg.g:(h + 1) * cfg.g].astype(np.float64).mean(axis=0).astype(np.float32)
                gn = _rng(cfg.seed, _TAG_NOISE, b, h)
                noise = gn.standard_normal((pos.size, D), dtype=np.float32) * np.float32(cfg.needle_noise)
                rows.append(f32_to_bf16_bits(np.float32(cfg.needle_amp) * qbar[None, :] + noise))
                at.append(pos + (b * cfg.Hkv + h) * T)
    if at:
        K.view(n, D)[torch.from_numpy(np.concatenate(at)).to(device)] = \
            torch.from_numpy(np.concatenate(rows).view(np.int16)).to(device).view(torch.bfloat16)
    seq_len = np.full((B,), cfg.L, dtype=np.int32)
    return Case(cfg, tuple(range(B)), basis, key_scale, q, K, V, None, None, seq_len, needles)


_TAG_REFIT = 100


def make_refit_keys(B: int, Hkv: int, T: int, seed: int, tau: float = 24.0, gap: float = 0.5):
    """bf16 keys [B][Hkv][T][128] with a planted spectrum, standing in for keys
    captured from a model (a basis refit needs keys with structure; N(0,1)
    keys are isotropic).  Per KV head: x = U (sigma * z), z ~ N(0, I), U a
    seeded random orthogonal matrix, sigma_i = exp(-i / tau) for i < 64 and
    gap * exp(-i / tau) beyond.  Returns (K bits, U [Hkv][128][128], sigma)."""
    D = 128
    i = np.arange(D)
    sigma = np.exp(-i / tau) * np.where(i < 64, 1.0, gap)
    U = np.stack([np.linalg.qr(_rng(seed, _TAG_REFIT, h).standard_normal((D, D)))[0]
                  for h in range(Hkv)])
    K = np.empty((B, Hkv, T, D), np.uint16)
    for b in range(B):
        for h in range(Hkv):
            z = _rng(seed, _TAG_REFIT + 1, b, h).standard_normal((T, D))
            K[b, h] = f32_to_bf16_bits(((z * sigma) @ U[h].T).astype(np.float32))
    return K, U, sigma

