"""ctypes binding of libsks (include/sks.h): argument marshalling only.

Every function here forwards torch tensors' device pointers and the current
HIP stream to the C ABI of the same name; all computation happens in the HIP
kernels.  The library is loaded after torch so that both share one HIP
runtime.  There is no fallback: a missing library raises.

The C ABI checks what a pointer can tell (NULL, alignment) but not how much
memory lies behind it, so every tensor is checked here first, before the
call: contiguous, on the GPU (or pinned host memory where a host tier
allows it) and exactly the byte size its layout in sks.h needs for this
cache and these parameters.  A mismatch raises ValueError and launches
nothing.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_LIB = None
LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsks.so")

SKS_OK, SKS_ERR_ARG, SKS_ERR_UNSUPPORTED, SKS_ERR_WORKSPACE, SKS_ERR_HIP = range(5)
KV_BF16, KV_I8, KV_I4 = 0, 1, 2
APPEND = -1
HEAD_DIM, RANK = 128, 64

TOPK_HIST_READY = 1
STEP_APPEND = 1
STEP_DENSE = 2
STEP_NO_SCORES = 4
CAND_KEEP_ESTIMATE = 1
CAND_TEST_HIGH = 2
CAND_TEST_ZERO = 4

EXPORTS = ("sks_last_error", "sks_runtime_version", "sks_workspace_bytes", "sks_workspace_init",
           "sks_sketch_build", "sks_sketch_build_query", "sks_sketch_score", "sks_topk_select",
           "sks_score_candidates", "sks_topk_select_candidates", "sks_gather_pack",
           "sks_sparse_decode_attn", "sks_decode_step", "sks_decode_step_static",
           "sks_refit_workspace_bytes", "sks_refit_gram", "sks_refit_basis",
           "sks_refit_key_scale")


class SksError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"sks error {code}: {msg}")
        self.code = code


class KVDesc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("Hkv", ctypes.c_int32), ("D", ctypes.c_int32),
                ("T_max", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("K", ctypes.c_void_p), ("V", ctypes.c_void_p),
                ("K_scale", ctypes.c_void_p), ("V_scale", ctypes.c_void_p),
                ("seq_len", ctypes.c_void_p),
                ("K_hot", ctypes.c_void_p), ("V_hot", ctypes.c_void_p),
                ("K_hot_scale", ctypes.c_void_p), ("V_hot_scale", ctypes.c_void_p),
                ("W_hot", ctypes.c_int32)]


class Params(ctypes.Structure):
    _fields_ = [("window", ctypes.c_int32), ("topk", ctypes.c_int32), ("pool", ctypes.c_int32),
                ("rank", ctypes.c_int32), ("rows", ctypes.c_int32)]


class StepDesc(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("Hq", ctypes.c_int32), ("basis", ctypes.c_void_p),
                ("basis_per_head", ctypes.c_int32), ("key_scale", ctypes.c_void_p),
                ("S", ctypes.c_void_p), ("Kp", ctypes.c_void_p), ("Vp", ctypes.c_void_p),
                ("sm_scale", ctypes.c_float), ("qsk", ctypes.c_void_p), ("qscale", ctypes.c_void_p),
                ("scores", ctypes.c_void_p), ("idx", ctypes.c_void_p), ("n_sel", ctypes.c_void_p),
                ("out", ctypes.c_void_p), ("lse", ctypes.c_void_p)]


def params(window: int, topk: int, pool: int = 1, rows: int = 1, rank: int = RANK) -> Params:
    return Params(window, topk, pool, rank, rows)


def lib():
    """Load libsks.so (built in-tree by build.py); raise if it is missing."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -m "
                               "long_context_sparse_sketch_amd.build` first")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        kvp, pp = ctypes.POINTER(KVDesc), ctypes.POINTER(Params)
        L.sks_last_error.restype = ctypes.c_char_p
        L.sks_last_error.argtypes = []
        L.sks_runtime_version.restype = i32
        L.sks_runtime_version.argtypes = []
        L.sks_workspace_bytes.restype = sz
        L.sks_workspace_bytes.argtypes = [kvp, pp, i32]
        L.sks_workspace_init.restype = ctypes.c_int
        L.sks_workspace_init.argtypes = [vp, sz, vp]
        L.sks_sketch_build.restype = ctypes.c_int
        L.sks_sketch_build.argtypes = [kvp, pp, vp, i32, vp, i32, i32, vp, vp, vp, vp]
        L.sks_sketch_build_query.restype = ctypes.c_int
        L.sks_sketch_build_query.argtypes = [vp, i32, i32, i32, i32, vp, i32, vp, vp, vp]
        L.sks_sketch_score.restype = ctypes.c_int
        L.sks_sketch_score.argtypes = [vp, vp, kvp, pp, vp, vp, sz, vp]
        L.sks_topk_select.restype = ctypes.c_int
        L.sks_topk_select.argtypes = [vp, kvp, pp, i32, vp, vp, vp, sz, vp]
        L.sks_score_candidates.restype = ctypes.c_int
        L.sks_score_candidates.argtypes = [vp, vp, kvp, pp, i32, vp, sz, vp]
        L.sks_topk_select_candidates.restype = ctypes.c_int
        L.sks_topk_select_candidates.argtypes = [vp, vp, kvp, pp, vp, vp, vp, vp, sz, vp]
        L.sks_gather_pack.restype = ctypes.c_int
        L.sks_gather_pack.argtypes = [kvp, pp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.sks_sparse_decode_attn.restype = ctypes.c_int
        L.sks_sparse_decode_attn.argtypes = [vp, i32, kvp, pp, vp, vp, vp, ctypes.c_float, vp,
                                             vp, vp, sz, vp]
        L.sks_decode_step.restype = ctypes.c_int
        L.sks_decode_step.argtypes = [kvp, pp, ctypes.POINTER(StepDesc), i32, vp, sz, vp]
        L.sks_decode_step_static.restype = ctypes.c_int
        L.sks_decode_step_static.argtypes = [kvp, pp, ctypes.POINTER(StepDesc), i32, vp]
        L.sks_refit_workspace_bytes.restype = sz
        L.sks_refit_workspace_bytes.argtypes = [kvp, i32, i32]
        L.sks_refit_gram.restype = ctypes.c_int
        L.sks_refit_gram.argtypes = [kvp, i32, i32, i32, vp, vp, sz, vp]
        L.sks_refit_basis.restype = ctypes.c_int
        L.sks_refit_basis.argtypes = [vp, i32, vp, vp, vp, sz, vp]
        L.sks_refit_key_scale.restype = ctypes.c_int
        L.sks_refit_key_scale.argtypes = [kvp, i32, i32, vp, i32, vp, vp, sz, vp]
        # the HIP runtime the library runs on (one of its dependencies)
        L.hipHostGetDevicePointer.restype = ctypes.c_int
        L.hipHostGetDevicePointer.argtypes = [ctypes.POINTER(vp), vp, ctypes.c_uint]
        _LIB = L
    return _LIB


def last_error() -> str:
    return lib().sks_last_error().decode()


def _check(rc: int):
    if rc != SKS_OK:
        raise SksError(rc, last_error())


def ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _nbytes(t) -> int:
    return 0 if t is None else t.numel() * t.element_size()


class _T:
    """One tensor argument: its name, the bytes its layout needs, whether it
    may be None and whether pinned host memory is allowed."""
    __slots__ = ("t", "name", "nbytes", "optional", "host_ok")

    def __init__(self, t, name: str, nbytes: int, optional: bool = False, host_ok: bool = False):
        self.t, self.name, self.nbytes = t, name, nbytes
        self.optional, self.host_ok = optional, host_ok


def _ptrs(*args: _T, stream=None, launch: bool = True, cache=None):
    """Device pointers of the arguments, after checking every one of them:
    first that each is present (unless optional), contiguous and exactly
    its layout's byte size, then that each is on the GPU (or pinned host
    memory where allowed), all on one device with `cache`'s lengths -- for
    a launch, the device of `stream` (the current device when it is None).  Raises ValueError naming
    the first argument that fails; nothing is launched."""
    for a in args:
        t = a.t
        if t is None:
            if not a.optional:
                raise ValueError(f"{a.name} is required")
            continue
        if not t.is_contiguous():
            raise ValueError(f"{a.name} must be contiguous")
        if _nbytes(t) != a.nbytes:
            raise ValueError(f"{a.name}: {a.nbytes} bytes expected, got {_nbytes(t)} "
                             f"(shape {tuple(t.shape)}, {t.dtype})")
    out = []
    for a in args:
        t = a.t
        if t is None:
            out.append(None)
        elif t.is_cuda:
            out.append(t.data_ptr())
        elif a.host_ok:
            out.append(device_address(t))
        else:
            raise ValueError(f"{a.name} must be a GPU tensor")
    devs = {(a.name, a.t.device.index) for a in args if a.t is not None and a.t.is_cuda}
    sl = getattr(cache, "seq_len", None)
    if sl is not None and sl.is_cuda:
        devs.add(("the cache", sl.device.index))
    idxs = {i for _, i in devs}
    if len(idxs) > 1:
        raise ValueError("tensors on several devices: "
                         + ", ".join(f"{n} on cuda:{i}" for n, i in sorted(devs)))
    if launch and idxs:
        dev = next(iter(idxs))
        want = getattr(stream, "device", None)
        want = torch.cuda.current_device() if stream is None else getattr(want, "index", dev)
        if want != dev:
            raise ValueError(f"tensors are on cuda:{dev} but the launch goes to cuda:{want} "
                             f"(use torch.cuda.device({dev}) or a stream of that device)")
    return out


def _row_bytes(dtype: int) -> int:
    return {KV_BF16: 2 * HEAD_DIM, KV_I8: HEAD_DIM, KV_I4: HEAD_DIM // 2}[dtype]


def device_address(t) -> int | None:
    """Address under which the GPU reaches tensor `t`: its data pointer for a
    device tensor; for a pinned host tensor the device address of its pinned
    allocation (hipHostGetDevicePointer) plus the tensor's offset in it."""
    if t is None:
        return None
    if t.is_cuda:
        return t.data_ptr()
    if not t.is_pinned():
        raise ValueError("a host tensor handed to the GPU must be pinned (pin_memory=True)")
    base = t.untyped_storage().data_ptr()
    dev = ctypes.c_void_p()
    rc = lib().hipHostGetDevicePointer(ctypes.byref(dev), ctypes.c_void_p(base), 0)
    if rc != 0 or not dev.value:
        raise SksError(SKS_ERR_HIP, f"hipHostGetDevicePointer failed ({rc})")
    return dev.value + (t.data_ptr() - base)


def _stream(stream):
    if stream is not None:
        return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream
    return torch.cuda.current_stream().cuda_stream


class Cache:
    """Descriptor of one layer's KV cache; keeps the tensors alive.

    K, V (and scales) may be device tensors or, with a hot tier, pinned host
    tensors.  hot = (K_hot, V_hot, K_hot_scale, V_hot_scale): the ring of the
    last W_hot positions in device memory, [B][Hkv][W_hot][row], position p
    in slot p % W_hot (scales None for bf16)."""

    def __init__(self, K, V, seq_len, K_scale=None, V_scale=None, hot=None):
        self.K, self.V, self.seq_len, self.K_scale, self.V_scale = K, V, seq_len, K_scale, V_scale
        self.hot = hot
        if K.dim() != 4:
            raise ValueError(f"K must be [B][Hkv][T][row], got shape {tuple(K.shape)}")
        B, Hkv, T, D = K.shape
        # bf16 rows as torch.bfloat16; int8 codes as torch.int8; packed int4
        # rows (64 bytes) as torch.uint8
        dtype = {torch.bfloat16: KV_BF16, torch.int8: KV_I8, torch.uint8: KV_I4}.get(K.dtype)
        if dtype is None:
            raise ValueError(f"K must be bfloat16, int8 or uint8 (packed int4), got {K.dtype}")
        if dtype == KV_I4:
            D *= 2
        if V.dtype != K.dtype:
            raise ValueError(f"V ({V.dtype}) must have K's dtype ({K.dtype})")
        rb, quant = K.shape[3] * K.element_size(), dtype != KV_BF16
        kv_b, sc_b = B * Hkv * T * rb, B * Hkv * T * 2
        if quant == (K_scale is None) or quant == (V_scale is None):
            raise ValueError("int8 / int4 caches need K_scale and V_scale, bf16 caches none")
        # K, V and their scales may be pinned host memory (read through its
        # device address: a host tier keeps the window in the device ring)
        args = [_T(K, "K", kv_b, host_ok=True), _T(V, "V", kv_b, host_ok=True),
                _T(K_scale, "K_scale", sc_b, optional=True, host_ok=True),
                _T(V_scale, "V_scale", sc_b, optional=True, host_ok=True),
                _T(seq_len, "seq_len", 4 * B)]
        W_hot = 0
        if hot is not None:
            hk, hv, hks, hvs = hot
            if hk is None or hk.dim() != 4:
                raise ValueError("K_hot must be [B][Hkv][W_hot][row]")
            if quant == (hks is None) or quant == (hvs is None):
                raise ValueError("a hot tier of an int8 / int4 cache needs its scales, bf16 none")
            W_hot = hk.shape[2]
            args += [_T(hk, "K_hot", B * Hkv * W_hot * rb), _T(hv, "V_hot", B * Hkv * W_hot * rb),
                     _T(hks, "K_hot_scale", B * Hkv * W_hot * 2, optional=True),
                     _T(hvs, "V_hot_scale", B * Hkv * W_hot * 2, optional=True)]
        ptrs = _ptrs(*args, launch=False) + [None] * (4 if hot is None else 0)
        self.desc = KVDesc(B, Hkv, D, T, dtype, *ptrs[:5], *ptrs[5:9], W_hot)

    @property
    def ref(self):
        return ctypes.byref(self.desc)


class _Dims:
    """The byte sizes of a call's tensors, from the cache descriptor and parameters."""

    def __init__(self, cache: Cache, p: Params | None = None):
        d = cache.desc
        self.B, self.Hkv, self.T = d.B, d.Hkv, d.T_max
        self.rb = _row_bytes(d.dtype) if d.D == HEAD_DIM else 0
        if p is not None:
            self.R, self.k, self.pool = p.rows, p.topk, max(1, p.pool)
            self.NB = self.T // self.pool
            self.C = p.topk + p.window + self.pool - 1

    def seg(self, per=1):            # [B][R][Hkv] x `per` bytes
        return self.B * self.R * self.Hkv * per

    def basis(self, basis, per_head):
        return _T(basis, "basis", (self.Hkv if per_head else 1) * RANK * HEAD_DIM * 4)

    def key_scale(self, ks):
        return _T(ks, "key_scale", 4 * self.Hkv)

    def S(self, S):                  # [B][Hkv][NB][64] int8
        return _T(S, "S", self.B * self.Hkv * self.NB * RANK)

    def pooled(self, t, name):       # Kp, Vp: [B][Hkv][NB][128] bf16, None when pool == 1
        return _T(t, name, self.B * self.Hkv * self.NB * HEAD_DIM * 2, optional=True)

    def scores(self, t):
        return _T(t, "scores", self.seg(4 * self.NB))

    def idx(self, t):
        return _T(t, "idx", self.seg(4 * self.k))

    def q(self, q):                  # [B][R][Hq][128] bf16; returns (arg, Hq)
        if q is None or q.dim() != 4 or q.shape[3] != HEAD_DIM:
            raise ValueError(f"q must be [B][R][Hq][{HEAD_DIM}] bf16")
        return _T(q, "q", self.B * self.R * q.shape[2] * HEAD_DIM * 2), q.shape[2]


def _ws(ws, optional=False):
    """A workspace: any contiguous GPU byte buffer (the library checks its size)."""
    return _T(ws, "ws", _nbytes(ws), optional=optional)


def workspace_bytes(cache: Cache, p: Params, Hq: int) -> int:
    return lib().sks_workspace_bytes(cache.ref, ctypes.byref(p), Hq)


def workspace_init(ws, stream=None):
    (wa,) = _ptrs(_ws(ws), stream=stream)
    _check(lib().sks_workspace_init(wa, _nbytes(ws), _stream(stream)))


def sketch_build(cache: Cache, p: Params, basis, key_scale, S, t_begin=0, t_end=None, Kp=None,
                 Vp=None, basis_per_head=False, stream=None):
    if t_end is None:
        t_end = cache.desc.T_max
    d = _Dims(cache, p)
    ba, ka, sa, kpa, vpa = _ptrs(d.basis(basis, basis_per_head), d.key_scale(key_scale), d.S(S),
                                 d.pooled(Kp, "Kp"), d.pooled(Vp, "Vp"), stream=stream, cache=cache)
    _check(lib().sks_sketch_build(cache.ref, ctypes.byref(p), ba, int(basis_per_head), ka,
                                  t_begin, t_end, sa, kpa, vpa, _stream(stream)))


def sketch_build_query(q, Hkv: int, basis, qsk, qscale=None, basis_per_head=False, stream=None):
    if q is None or q.dim() != 4 or q.shape[3] != HEAD_DIM:
        raise ValueError(f"q must be [B][R][Hq][{HEAD_DIM}] bf16")
    B, R, Hq, _ = q.shape
    qa, ba, qsa, qca = _ptrs(_T(q, "q", B * R * Hq * HEAD_DIM * 2),
                             _T(basis, "basis",
                                (Hkv if basis_per_head else 1) * RANK * HEAD_DIM * 4),
                             _T(qsk, "qsk", B * R * Hkv * RANK),
                             _T(qscale, "qscale", 4 * B * R * Hkv, optional=True), stream=stream)
    _check(lib().sks_sketch_build_query(qa, B, R, Hq, Hkv, ba, int(basis_per_head), qsa, qca,
                                        _stream(stream)))


def sketch_score(qsk, S, cache: Cache, p: Params, scores, ws=None, stream=None):
    d = _Dims(cache, p)
    qa, sa, ca, wa = _ptrs(_T(qsk, "qsk", d.seg(RANK)), d.S(S), d.scores(scores),
                           _ws(ws, optional=True), stream=stream, cache=cache)
    _check(lib().sks_sketch_score(qa, sa, cache.ref, ctypes.byref(p), ca, wa, _nbytes(ws),
                                  _stream(stream)))


def topk_select(scores, cache: Cache, p: Params, idx, n_sel, ws, hist_ready=False, stream=None):
    d = _Dims(cache, p)
    ca, ia, na, wa = _ptrs(d.scores(scores), d.idx(idx),
                           _T(n_sel, "n_sel", d.seg(4), optional=True), _ws(ws), stream=stream,
                           cache=cache)
    _check(lib().sks_topk_select(ca, cache.ref, ctypes.byref(p),
                                 TOPK_HIST_READY if hist_ready else 0, ia, na, wa, _nbytes(ws),
                                 _stream(stream)))


def score_candidates(qsk, S, cache: Cache, p: Params, ws, flags=0, stream=None):
    """Candidate mode's score pass (sample estimate unless CAND_KEEP_ESTIMATE)."""
    d = _Dims(cache, p)
    qa, sa, wa = _ptrs(_T(qsk, "qsk", d.seg(RANK)), d.S(S), _ws(ws), stream=stream, cache=cache)
    _check(lib().sks_score_candidates(qa, sa, cache.ref, ctypes.byref(p), int(flags), wa,
                                      _nbytes(ws), _stream(stream)))


def topk_select_candidates(qsk, S, cache: Cache, p: Params, scores, idx, n_sel, ws,
                           stream=None):
    """Selection from score_candidates' lists; `scores` is scratch."""
    d = _Dims(cache, p)
    qa, sa, ca, ia, na, wa = _ptrs(_T(qsk, "qsk", d.seg(RANK)), d.S(S), d.scores(scores),
                                   d.idx(idx), _T(n_sel, "n_sel", d.seg(4), optional=True),
                                   _ws(ws), stream=stream, cache=cache)
    _check(lib().sks_topk_select_candidates(qa, sa, cache.ref, ctypes.byref(p), ca, ia, na, wa,
                                            _nbytes(ws), _stream(stream)))


def gather_pack(cache: Cache, p: Params, idx, K_out, V_out, n_out, Kp=None, Vp=None,
                Ks_out=None, Vs_out=None, stream=None):
    d = _Dims(cache, p)
    rows = d.seg(d.C * d.rb)
    ptrs = _ptrs(d.idx(idx), d.pooled(Kp, "Kp"), d.pooled(Vp, "Vp"), _T(K_out, "K_out", rows),
                 _T(V_out, "V_out", rows), _T(Ks_out, "Ks_out", d.seg(2 * d.C), optional=True),
                 _T(Vs_out, "Vs_out", d.seg(2 * d.C), optional=True),
                 _T(n_out, "n_out", d.seg(4)), stream=stream, cache=cache)
    _check(lib().sks_gather_pack(cache.ref, ctypes.byref(p), *ptrs, _stream(stream)))


def sparse_decode_attn(q, cache: Cache, p: Params, idx, out, ws, lse=None, Kp=None, Vp=None,
                       sm_scale=None, stream=None):
    d = _Dims(cache, p)
    qt, Hq = d.q(q)
    sm = 1.0 / math.sqrt(HEAD_DIM) if sm_scale is None else sm_scale
    qa, ia, kpa, vpa, oa, la, wa = _ptrs(
        qt, d.idx(idx), d.pooled(Kp, "Kp"), d.pooled(Vp, "Vp"),
        _T(out, "out", d.B * d.R * Hq * HEAD_DIM * 4),
        _T(lse, "lse", d.B * d.R * Hq * 4, optional=True), _ws(ws), stream=stream, cache=cache)
    _check(lib().sks_sparse_decode_attn(qa, Hq, cache.ref, ctypes.byref(p), ia, kpa, vpa,
                                        ctypes.c_float(sm), oa, la, wa, _nbytes(ws),
                                        _stream(stream)))


def decode_step(cache: Cache, p: Params, q, basis, key_scale, S, qsk, scores, idx, out, ws,
                qscale=None, n_sel=None, lse=None, Kp=None, Vp=None, sm_scale=None,
                basis_per_head=False, append=True, dense=False, keep_scores=True, stream=None):
    """The whole decode step (append, query sketch, score, select, attend) in one call;
    dense: no scoring or selection, attend the last window + topk tokens;
    keep_scores=False: `scores` is scratch (candidate mode where it pays)."""
    d = _Dims(cache, p)
    qt, Hq = d.q(q)
    sm = 1.0 / math.sqrt(HEAD_DIM) if sm_scale is None else sm_scale
    (qa, ba, ka, sa, kpa, vpa, qsa, qca, ca, ia, na, oa, la, wa) = _ptrs(
        qt, d.basis(basis, basis_per_head), d.key_scale(key_scale), d.S(S),
        d.pooled(Kp, "Kp"), d.pooled(Vp, "Vp"), _T(qsk, "qsk", d.seg(RANK)),
        _T(qscale, "qscale", d.seg(4), optional=True), d.scores(scores), d.idx(idx),
        _T(n_sel, "n_sel", d.seg(4), optional=True),
        _T(out, "out", d.B * d.R * Hq * HEAD_DIM * 4),
        _T(lse, "lse", d.B * d.R * Hq * 4, optional=True), _ws(ws), stream=stream, cache=cache)
    st = StepDesc(qa, Hq, ba, int(basis_per_head), ka, sa, kpa, vpa, sm, qsa, qca, ca, ia, na,
                  oa, la)
    _check(lib().sks_decode_step(cache.ref, ctypes.byref(p), ctypes.byref(st),
                                 (STEP_APPEND if append else 0) | (STEP_DENSE if dense else 0)
                                 | (0 if keep_scores else STEP_NO_SCORES),
                                 wa, _nbytes(ws), _stream(stream)))


STATIC_WORKSPACE_BYTES = 96 << 20      # SKS_STATIC_WORKSPACE_BYTES of sks.h


def decode_step_static(cache: Cache, p: Params, q, basis, key_scale, S, qsk, scores, idx, out,
                       qscale=None, n_sel=None, lse=None, Kp=None, Vp=None, sm_scale=None,
                       basis_per_head=False, append=True, dense=False, keep_scores=True,
                       stream=None):
    """decode_step with the library's static workspace (sks_decode_step_static):
    no workspace argument, nothing allocated by the call."""
    d = _Dims(cache, p)
    qt, Hq = d.q(q)
    sm = 1.0 / math.sqrt(HEAD_DIM) if sm_scale is None else sm_scale
    (qa, ba, ka, sa, kpa, vpa, qsa, qca, ca, ia, na, oa, la) = _ptrs(
        qt, d.basis(basis, basis_per_head), d.key_scale(key_scale), d.S(S),
        d.pooled(Kp, "Kp"), d.pooled(Vp, "Vp"), _T(qsk, "qsk", d.seg(RANK)),
        _T(qscale, "qscale", d.seg(4), optional=True), d.scores(scores), d.idx(idx),
        _T(n_sel, "n_sel", d.seg(4), optional=True),
        _T(out, "out", d.B * d.R * Hq * HEAD_DIM * 4),
        _T(lse, "lse", d.B * d.R * Hq * 4, optional=True), stream=stream, cache=cache)
    st = StepDesc(qa, Hq, ba, int(basis_per_head), ka, sa, kpa, vpa, sm, qsa, qca, ca, ia, na,
                  oa, la)
    _check(lib().sks_decode_step_static(cache.ref, ctypes.byref(p), ctypes.byref(st),
                                        (STEP_APPEND if append else 0)
                                        | (STEP_DENSE if dense else 0)
                                        | (0 if keep_scores else STEP_NO_SCORES),
                                        _stream(stream)))


def refit_workspace_bytes(cache: Cache, t_begin: int, t_end: int) -> int:
    return lib().sks_refit_workspace_bytes(cache.ref, t_begin, t_end)


def refit_gram(cache: Cache, t_begin: int, t_end: int, gram, ws, per_head=True, stream=None):
    n = cache.desc.Hkv if per_head else 1
    ga, wa = _ptrs(_T(gram, "gram", n * HEAD_DIM * HEAD_DIM * 8), _ws(ws), stream=stream,
                   cache=cache)
    _check(lib().sks_refit_gram(cache.ref, t_begin, t_end, int(per_head), ga, wa, _nbytes(ws),
                                _stream(stream)))


def refit_basis(gram, basis, ws, eigval=None, stream=None):
    if gram is None or gram.dim() != 3:
        raise ValueError(f"gram must be [n][{HEAD_DIM}][{HEAD_DIM}] float64")
    n = gram.shape[0]
    ga, ba, ea, wa = _ptrs(_T(gram, "gram", n * HEAD_DIM * HEAD_DIM * 8),
                           _T(basis, "basis", n * RANK * HEAD_DIM * 4),
                           _T(eigval, "eigval", n * HEAD_DIM * 8, optional=True), _ws(ws),
                           stream=stream)
    _check(lib().sks_refit_basis(ga, n, ba, ea, wa, _nbytes(ws), _stream(stream)))


def refit_key_scale(cache: Cache, t_begin: int, t_end: int, basis, key_scale, ws,
                    basis_per_head=True, stream=None):
    d = _Dims(cache)
    ba, ka, wa = _ptrs(d.basis(basis, basis_per_head), d.key_scale(key_scale), _ws(ws),
                       stream=stream, cache=cache)
    _check(lib().sks_refit_key_scale(cache.ref, t_begin, t_end, ba, int(basis_per_head), ka, wa,
                                     _nbytes(ws), _stream(stream)))
