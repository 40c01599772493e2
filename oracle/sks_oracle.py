"""CPU oracle for sparse-sketch decode attention.  TEST INFRASTRUCTURE ONLY.

Only the tests, the package's smoke check and the benchmark's CPU-baseline leg
may import this module.  It shares no code with the HIP path (no kernels,
headers, helpers or constants) and imports nothing from it; both sides are fed
the same seeded inputs by the synthetic-input module.

Plain NumPy, float64 for real arithmetic and int64 for integers, loops over
(sequence, query row, KV head).  What it computes, and where it comes from:

* Key sketch -- "8 agents x 250K context, concurrently, on two 3090s", claims
  list (every decode step each attention layer reads ~1% of the tokens, picked
  with a tiny rank-64 key sketch) and "What it took" (kernels that build the
  sketch; a frozen sketch basis stored in one file).  Read as a linear
  projection y = P k onto 64 orthonormal basis vectors, quantized to int8 with
  a scale fixed per KV head and frozen with the basis.
* Query sketch -- same passage; under grouped-query attention the query side
  uses the mean of the KV head's group of query vectors, quantized with its
  own absmax/127 scale.
* Scores -- "What it took": score every token.  Exact integer dot product of
  the two int8 sketches.
* Top-k -- "What it took": pick the top ~2K.  The k largest scores of the far
  region, lower index first among equal scores, emitted in ascending order.
* Window and merged softmax -- "Agens SGLang" README, "What it adds": a
  4,096-token sliding window plus a 4:1 mean-pooled far field, merged under
  one softmax.  The window is the last W positions and is always attended;
  selection is over the region before it, so the two sets are disjoint.
* Pooled far field -- same passage: r consecutive tokens aligned to position
  0 are averaged (K and V), stored as bfloat16, and sketched from the stored
  pooled key; a tail shorter than r joins the exact window; pooled logits get
  no count bias.
* Basis refit -- "8 agents x 250K context ...", "What it took": a frozen
  sketch basis in one file plus a script that refits it.  Read as principal
  directions of captured keys: the Gram matrix G = sum_t x_t x_t^T of the
  keys, its 64 leading eigenvectors (largest eigenvalues first, each signed so
  that its largest-magnitude component is positive) as the basis rows, and a
  key scale max_t max_c |(P x_t)_c| / 127, so that no captured key's code
  clips.
* Verify rows -- "Agens SGLang", "Quick start": the verify step of speculative
  decoding is served as a chain.  Row i of a sequence sits at position L-1+i,
  sees [0, L+i) and has its own window and its own selection, so verifying is
  the same as decoding the rows one by one.

Every function here is pinned by tests/test_oracle_pins.py (closed forms,
hand-worked examples in tests/golden/, brute force on tiny inputs, reduction
to torch's dense attention, invariants), and tests/test_oracle_mutations.py
shows that planted mistakes are caught.  The pages print no worked example of
their own, so no value here is checked against a printed number.
"""
from __future__ import annotations

import math

import numpy as np

CODE_MAX = 127          # symmetric int8 codes, -128 unused
SCORE_BOUND = 64 * CODE_MAX * CODE_MAX


# --------------------------------------------------------------------------
# storage formats -> float64 (exact)
# --------------------------------------------------------------------------
def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> exact float64 values."""
    u32 = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u32.view(np.float32).astype(np.float64)


def f16_to_f64(bits: np.ndarray) -> np.ndarray:
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def i8_rows_to_f64(codes: np.ndarray, scale_bits: np.ndarray) -> np.ndarray:
    """int8 row codes times the row's fp16 scale, exactly."""
    return np.asarray(codes, dtype=np.int8).astype(np.float64) * f16_to_f64(scale_bits)[..., None]


def i4_unpack(packed: np.ndarray) -> np.ndarray:
    """int4 rows [..][64] uint8 -> codes [..][128] int64.

    Byte j of a row holds dimension 2j in its low nibble and dimension 2j+1
    in its high nibble; each nibble is a two's-complement code in [-8, 7].
    (The int4 cache of the claims list of "8 agents x 250K context ...": the
    pages give no bit layout, so this plain one is the reading.)"""
    p = np.asarray(packed, dtype=np.uint8).astype(np.int64)
    lo, hi = p & 0xF, p >> 4
    lo = np.where(lo >= 8, lo - 16, lo)
    hi = np.where(hi >= 8, hi - 16, hi)
    return np.stack([lo, hi], axis=-1).reshape(*p.shape[:-1], 2 * p.shape[-1])


def i4_rows_to_f64(packed: np.ndarray, scale_bits: np.ndarray) -> np.ndarray:
    """int4 row codes times the row's fp16 scale, exactly."""
    return i4_unpack(packed).astype(np.float64) * f16_to_f64(scale_bits)[..., None]


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 value, ties to even.

    bfloat16 keeps 8 significant bits: write x = m * 2^e with 0.5 <= |m| < 1,
    round m * 2^8 to an integer (half to even) and scale back.  Normal range
    only (the pooled means of the synthetic caches never leave it).
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    return np.ldexp(np.rint(m * 256.0) / 256.0, e)


def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Bit pattern of values that are already exactly representable in bf16."""
    f32 = np.asarray(x, dtype=np.float64).astype(np.float32)
    return (f32.view(np.uint32) >> 16).astype(np.uint16)


# --------------------------------------------------------------------------
# sketches
# --------------------------------------------------------------------------
def quantize_codes(y: np.ndarray, scale) -> np.ndarray:
    """code = clamp(round_half_even(y / scale), -127, 127) as int8."""
    return np.clip(np.rint(np.asarray(y, np.float64) / scale), -CODE_MAX, CODE_MAX).astype(np.int8)


def project(x: np.ndarray, basis: np.ndarray) -> np.ndarray:
    """y = P x for each row x: coordinates on the 64 basis vectors (rows of `basis`)."""
    return np.asarray(x, np.float64) @ np.asarray(basis, np.float64).T


def key_sketch(keys: np.ndarray, basis: np.ndarray, key_scale: float):
    """Rank-64 int8 sketch of cached keys ([n][128] float64) -> (y, codes)."""
    y = project(keys, basis)
    return y, quantize_codes(y, float(key_scale))


def pool_mean(x: np.ndarray, r: int) -> np.ndarray:
    """4:1 (generally r:1) mean of consecutive rows aligned to 0, rounded to bf16.

    r == 1 means no pooling and returns the rows unchanged.

    Returns float64 values that are exactly representable in bfloat16, one row
    per complete block (a trailing partial block is dropped).
    """
    x = np.asarray(x, np.float64)
    nb = x.shape[0] // r
    if r == 1:
        return x.copy()           # no pooling: the cached rows themselves
    return round_to_bf16(x[: nb * r].reshape(nb, r, x.shape[1]).mean(axis=1))


def query_sketch(q_group: np.ndarray, basis: np.ndarray):
    """Sketch of one KV head's query group ([g][128] float64).

    qbar = mean of the group; y = P qbar; scale = max|y| / 127 (0 if y == 0);
    codes = clamp(rne(y / scale)), all zero when scale is 0.
    Returns (codes int8[64], scale float, y float64[64]).
    """
    qbar = np.asarray(q_group, np.float64).mean(axis=0)
    y = project(qbar[None, :], basis)[0]
    amax = float(np.abs(y).max()) if y.size else 0.0
    if amax == 0.0:
        return np.zeros(y.shape, np.int8), 0.0, y
    scale = amax / CODE_MAX
    return quantize_codes(y, scale), scale, y


def scores(qcode: np.ndarray, kcodes: np.ndarray) -> np.ndarray:
    """Exact int64 dot of the query code with every key code row."""
    s = np.asarray(kcodes, np.int64) @ np.asarray(qcode, np.int64)
    assert np.all(np.abs(s) <= SCORE_BOUND)
    return s


# --------------------------------------------------------------------------
# selection and attention set
# --------------------------------------------------------------------------
def row_geometry(L_i: int, window: int, r: int):
    """(n_far, win_start) of a row of valid length L_i.

    The far region is [0, L_i - window) cut into whole r-blocks aligned to 0;
    n_far counts them (tokens when r == 1).  Everything from win_start =
    n_far * r to L_i is attended exactly (the window plus any tail shorter
    than r).  With L_i <= window nothing is far.
    """
    if L_i <= window:
        return 0, 0
    n_far = (L_i - window) // r
    return n_far, n_far * r


def select_topk(sc: np.ndarray, k: int) -> np.ndarray:
    """Indices of the min(k, n) largest scores; lower index wins ties; ascending."""
    sc = np.asarray(sc, np.int64)
    n = sc.shape[0]
    k_eff = min(k, n)
    order = np.lexsort((np.arange(n), -sc))      # primary: score desc, then index asc
    return np.sort(order[:k_eff]).astype(np.int64)


def pad_idx(sel: np.ndarray, k: int) -> np.ndarray:
    out = np.full((k,), -1, dtype=np.int64)
    out[: sel.shape[0]] = sel
    return out


def attend(q_heads: np.ndarray, Krows: np.ndarray, Vrows: np.ndarray, sm_scale: float):
    """One softmax over the attention set for each query head.

    z_j = (q . K_j) * sm_scale; p = softmax(z); out = sum_j p_j V_j;
    lse = log sum_j exp(z_j).  Empty set: out = 0, lse = -inf.
    """
    q = np.asarray(q_heads, np.float64)
    if Krows.shape[0] == 0:
        return np.zeros((q.shape[0], Vrows.shape[1] if Vrows.ndim == 2 else q.shape[1])), \
            np.full((q.shape[0],), -np.inf)
    z = (q @ np.asarray(Krows, np.float64).T) * sm_scale
    m = z.max(axis=1, keepdims=True)
    e = np.exp(z - m)
    l = e.sum(axis=1, keepdims=True)
    out = (e / l) @ np.asarray(Vrows, np.float64)
    lse = (m + np.log(l))[:, 0]
    return out, lse


# --------------------------------------------------------------------------
# one decode step
# --------------------------------------------------------------------------
KV_BF16, KV_I8, KV_I4 = 0, 1, 2      # cache storage: bf16 rows, int8 codes, packed int4 codes


def cache_rows(K, V, Ks, Vs, b: int, h: int, kv_dtype: int, T: int | None = None):
    """Float64 K, V rows [T][128] of (sequence b, KV head h).

    kv_dtype: KV_BF16 (bf16 bits), KV_I8 (int8 codes, fp16-bit row scales
    Ks, Vs) or KV_I4 (packed int4 codes [..][64] uint8, fp16-bit row scales)."""
    T = K.shape[2] if T is None else T
    kv_dtype = int(kv_dtype)
    if kv_dtype == KV_I8:
        return (i8_rows_to_f64(K[b, h, :T], Ks[b, h, :T]),
                i8_rows_to_f64(V[b, h, :T], Vs[b, h, :T]))
    if kv_dtype == KV_I4:
        return (i4_rows_to_f64(K[b, h, :T], Ks[b, h, :T]),
                i4_rows_to_f64(V[b, h, :T], Vs[b, h, :T]))
    if kv_dtype != KV_BF16:
        raise ValueError(f"unknown KV storage {kv_dtype}")
    return bf16_to_f64(K[b, h, :T]), bf16_to_f64(V[b, h, :T])


def decode_head(qrows: np.ndarray, Kf: np.ndarray, Vf: np.ndarray, basis: np.ndarray,
                key_scale: float, L0: int, window: int, topk: int, r: int,
                sm_scale: float, codes=None):
    """Full step for one (sequence, KV head), every query row.

    qrows: [R][g][128] float64 query vectors of this KV head's group.
    Kf, Vf: [T][128] float64 cache rows (T >= L0 + R - 1).
    codes: optional (key codes [T / r][64], [query code [64] per row]) used in
    place of the sketches computed here (the scores, selection and attention
    are then those of the given codes; qscale is reported as nan).
    Returns a dict of per-row lists plus the key sketch of the cache.
    """
    R = qrows.shape[0]
    T = Kf.shape[0]
    Kp, Vp = pool_mean(Kf, r), pool_mean(Vf, r)       # pooled rows (r == 1: the rows)
    if codes is None:
        _, kcodes = key_sketch(Kp, basis, key_scale)  # one code row per block/token
    else:
        kcodes = np.asarray(codes[0], np.int8)
    res = {"kcodes": kcodes, "Kp": Kp, "Vp": Vp, "qcode": [], "qscale": [], "scores": [],
           "idx": [], "n_sel": [], "out": [], "lse": [], "n_far": [], "win_start": []}
    for i in range(R):
        Li = max(0, min(L0 + i, T))
        n_far, ws = row_geometry(Li, window, r)
        if codes is None:
            qc, qs, _ = query_sketch(qrows[i], basis)
        else:
            qc, qs = np.asarray(codes[1][i], np.int8), float("nan")
        sc = scores(qc, kcodes[:n_far])
        sel = select_topk(sc, topk)
        Kset = np.concatenate([Kp[sel], Kf[ws:Li]], axis=0)
        Vset = np.concatenate([Vp[sel], Vf[ws:Li]], axis=0)
        out, lse = attend(qrows[i], Kset, Vset, sm_scale)
        res["qcode"].append(qc)
        res["qscale"].append(qs)
        res["scores"].append(sc)
        res["idx"].append(pad_idx(sel, topk))
        res["n_sel"].append(sel.shape[0])
        res["out"].append(out)
        res["lse"].append(lse)
        res["n_far"].append(n_far)
        res["win_start"].append(ws)
    return res


def head_basis(basis: np.ndarray, h: int) -> np.ndarray:
    """The basis of KV head h: the one shared basis ([64][128]), or row h of a
    per-head basis ([Hkv][64][128])."""
    basis = np.asarray(basis, np.float64)
    return basis if basis.ndim == 2 else basis[h]


def head_key_scale(key_scale, h: int) -> float:
    """The frozen key-sketch scale of KV head h (one scale per KV head)."""
    return float(np.asarray(key_scale, np.float64)[h])


def decode_step(q, K, V, Ks, Vs, seq_len, basis, key_scale, window: int, topk: int,
                r: int, kv_dtype: int, heads=None, sm_scale: float | None = None, codes=None):
    """Oracle decode step over a batch.

    q: [B][R][Hq][128] bf16 bits; K, V: [B][Hkv][T][128] bf16 bits or int8, or
    [B][Hkv][T][64] packed int4 (see cache_rows), the codes with fp16-bit row
    scales Ks, Vs [B][Hkv][T]; seq_len [B] (row-0 lengths); basis
    [64][128] (shared) or [Hkv][64][128]; key_scale [Hkv].
    heads: optional iterable of (b, h) pairs to compute (default: all).
    codes: optional (key codes [B][Hkv][T / r][64], query codes [B][R][Hkv][64])
    int8 arrays used instead of the sketches this step would compute (for
    checking a selection made from another implementation's sketches).
    Returns {(b, h): decode_head result}.
    """
    B, R, Hq, D = q.shape
    Hkv = K.shape[1]
    g = Hq // Hkv
    sm = 1.0 / math.sqrt(D) if sm_scale is None else sm_scale
    qf = bf16_to_f64(q)
    pairs = [(b, h) for b in range(B) for h in range(Hkv)] if heads is None else list(heads)
    out = {}
    for b, h in pairs:
        Kf, Vf = cache_rows(K, V, Ks, Vs, b, h, kv_dtype)
        given = None if codes is None else (codes[0][b, h], [codes[1][b, i, h] for i in range(R)])
        out[(b, h)] = decode_head(qf[b, :, h * g:(h + 1) * g], Kf, Vf, head_basis(basis, h),
                                  head_key_scale(key_scale, h), int(seq_len[b]), window, topk,
                                  r, sm, codes=given)
    return out


# --------------------------------------------------------------------------
# sketch-basis refit
# --------------------------------------------------------------------------
def refit_keys(K, seq_len, h: int, t_begin: int, t_end: int) -> np.ndarray:
    """Captured keys of KV head h: positions [t_begin, min(t_end, L_b)) of
    every sequence b, bf16 bits -> float64 rows, sequences in order."""
    rows = []
    for b in range(K.shape[0]):
        hi = min(int(t_end), int(seq_len[b]), K.shape[2])
        lo = max(0, int(t_begin))
        if hi > lo:
            rows.append(bf16_to_f64(K[b, h, lo:hi]))
    return np.concatenate(rows, axis=0) if rows else np.zeros((0, K.shape[3]))


def key_gram(keys: np.ndarray) -> np.ndarray:
    """G = sum over keys x of the outer product x x^T ([n][128] -> [128][128])."""
    x = np.asarray(keys, np.float64)
    return x.T @ x


def basis_from_gram(G: np.ndarray, rank: int = 64):
    """The `rank` leading eigenvectors of the symmetric matrix G as rows
    (largest eigenvalue first; equal eigenvalues keep the solver's order),
    each signed so that its largest-magnitude component (the first one on
    ties) is positive.  Returns (basis [rank][128], eigenvalues [128]
    descending)."""
    w, U = np.linalg.eigh(np.asarray(G, np.float64))
    order = np.argsort(-w, kind="stable")
    w, U = w[order], U[:, order]
    P = U[:, :rank].T.copy()
    for r in range(rank):
        k = int(np.argmax(np.abs(P[r])))
        if P[r, k] < 0:
            P[r] = -P[r]
    return P, w


def refit_key_scale(keys: np.ndarray, basis: np.ndarray) -> float:
    """max over keys and sketch coordinates of |P x| / 127 (1.0 when every
    projection is zero, where any scale gives all-zero codes)."""
    if len(keys) == 0:
        return 1.0
    m = float(np.abs(project(keys, basis)).max())
    return m / CODE_MAX if m > 0 else 1.0


def refit(K, seq_len, t_begin: int, t_end: int, per_head: bool = True, rank: int = 64):
    """Refit from a bf16 cache: per KV head (or one basis from the keys of
    every head).  Returns (gram [n][128][128], basis [n][rank][128] float64,
    eigenvalues [n][128], key_scale [Hkv]) with n = Hkv or 1."""
    Hkv = K.shape[1]
    keys = [refit_keys(K, seq_len, h, t_begin, t_end) for h in range(Hkv)]
    grams = [key_gram(k) for k in keys]
    if not per_head:
        grams = [np.sum(grams, axis=0)]
    fits = [basis_from_gram(G, rank) for G in grams]
    basis = np.stack([f[0] for f in fits])
    eig = np.stack([f[1] for f in fits])
    scale = np.array([refit_key_scale(keys[h], basis[h if per_head else 0]) for h in range(Hkv)])
    return np.stack(grams), basis, eig, scale

