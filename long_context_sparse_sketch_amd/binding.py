"""ctypes binding of libsks (include/sks.h): argument marshalling only.

Every function here forwards torch tensors' device pointers and the current
HIP stream to the C ABI of the same name; all computation happens in the HIP
kernels.  The library is loaded after torch so that both share one HIP
runtime.  There is no fallback: a missing library raises.
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

EXPORTS = ("sks_last_error", "sks_runtime_version", "sks_workspace_bytes", "sks_workspace_init",
           "sks_sketch_build", "sks_sketch_build_query", "sks_sketch_score", "sks_topk_select",
           "sks_gather_pack", "sks_sparse_decode_attn", "sks_decode_step",
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
        L.sks_gather_pack.restype = ctypes.c_int
        L.sks_gather_pack.argtypes = [kvp, pp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.sks_sparse_decode_attn.restype = ctypes.c_int
        L.sks_sparse_decode_attn.argtypes = [vp, i32, kvp, pp, vp, vp, vp, ctypes.c_float, vp,
                                             vp, vp, sz, vp]
        L.sks_decode_step.restype = ctypes.c_int
        L.sks_decode_step.argtypes = [kvp, pp, ctypes.POINTER(StepDesc), i32, vp, sz, vp]
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
        B, Hkv, T, D = K.shape
        # int8 codes as torch.int8; packed int4 rows (64 bytes) as torch.uint8
        dtype = {torch.int8: KV_I8, torch.uint8: KV_I4}.get(K.dtype, KV_BF16)
        if dtype == KV_I4:
            D *= 2
        if hot is None:
            hk = hv = hks = hvs = None
            W_hot = 0
        else:
            hk, hv, hks, hvs = hot
            W_hot = hk.shape[2]
        da = device_address
        self.desc = KVDesc(B, Hkv, D, T, dtype, da(K), da(V), da(K_scale), da(V_scale),
                           ptr(seq_len), ptr(hk), ptr(hv), ptr(hks), ptr(hvs), W_hot)

    @property
    def ref(self):
        return ctypes.byref(self.desc)


def _nbytes(t) -> int:
    return 0 if t is None else t.numel() * t.element_size()


def workspace_bytes(cache: Cache, p: Params, Hq: int) -> int:
    return lib().sks_workspace_bytes(cache.ref, ctypes.byref(p), Hq)


def workspace_init(ws, stream=None):
    _check(lib().sks_workspace_init(ptr(ws), _nbytes(ws), _stream(stream)))


def sketch_build(cache: Cache, p: Params, basis, key_scale, S, t_begin=0, t_end=None, Kp=None,
                 Vp=None, basis_per_head=False, stream=None):
    if t_end is None:
        t_end = cache.desc.T_max
    _check(lib().sks_sketch_build(cache.ref, ctypes.byref(p), ptr(basis), int(basis_per_head),
                                  ptr(key_scale), t_begin, t_end, ptr(S), ptr(Kp), ptr(Vp),
                                  _stream(stream)))


def sketch_build_query(q, Hkv: int, basis, qsk, qscale=None, basis_per_head=False, stream=None):
    B, R, Hq, _ = q.shape
    _check(lib().sks_sketch_build_query(ptr(q), B, R, Hq, Hkv, ptr(basis), int(basis_per_head),
                                        ptr(qsk), ptr(qscale), _stream(stream)))


def sketch_score(qsk, S, cache: Cache, p: Params, scores, ws=None, stream=None):
    _check(lib().sks_sketch_score(ptr(qsk), ptr(S), cache.ref, ctypes.byref(p), ptr(scores),
                                  ptr(ws), _nbytes(ws), _stream(stream)))


def topk_select(scores, cache: Cache, p: Params, idx, n_sel, ws, hist_ready=False, stream=None):
    _check(lib().sks_topk_select(ptr(scores), cache.ref, ctypes.byref(p),
                                 TOPK_HIST_READY if hist_ready else 0, ptr(idx), ptr(n_sel),
                                 ptr(ws), _nbytes(ws), _stream(stream)))


def gather_pack(cache: Cache, p: Params, idx, K_out, V_out, n_out, Kp=None, Vp=None,
                Ks_out=None, Vs_out=None, stream=None):
    _check(lib().sks_gather_pack(cache.ref, ctypes.byref(p), ptr(idx), ptr(Kp), ptr(Vp),
                                 ptr(K_out), ptr(V_out), ptr(Ks_out), ptr(Vs_out), ptr(n_out),
                                 _stream(stream)))


def sparse_decode_attn(q, cache: Cache, p: Params, idx, out, ws, lse=None, Kp=None, Vp=None,
                       sm_scale=None, stream=None):
    Hq = q.shape[2]
    sm = 1.0 / math.sqrt(q.shape[3]) if sm_scale is None else sm_scale
    _check(lib().sks_sparse_decode_attn(ptr(q), Hq, cache.ref, ctypes.byref(p), ptr(idx),
                                        ptr(Kp), ptr(Vp), ctypes.c_float(sm), ptr(out), ptr(lse),
                                        ptr(ws), _nbytes(ws), _stream(stream)))


def decode_step(cache: Cache, p: Params, q, basis, key_scale, S, qsk, scores, idx, out, ws,
                qscale=None, n_sel=None, lse=None, Kp=None, Vp=None, sm_scale=None,
                basis_per_head=False, append=True, dense=False, stream=None):
    """The whole decode step (append, query sketch, score, select, attend) in one call;
    dense: no scoring or selection, attend the last window + topk tokens."""
    sm = 1.0 / math.sqrt(q.shape[3]) if sm_scale is None else sm_scale
    st = StepDesc(ptr(q), q.shape[2], ptr(basis), int(basis_per_head), ptr(key_scale), ptr(S),
                  ptr(Kp), ptr(Vp), sm, ptr(qsk), ptr(qscale), ptr(scores), ptr(idx), ptr(n_sel),
                  ptr(out), ptr(lse))
    _check(lib().sks_decode_step(cache.ref, ctypes.byref(p), ctypes.byref(st),
                                 (STEP_APPEND if append else 0) | (STEP_DENSE if dense else 0),
                                 ptr(ws), _nbytes(ws),
                                 _stream(stream)))


def refit_workspace_bytes(cache: Cache, t_begin: int, t_end: int) -> int:
    return lib().sks_refit_workspace_bytes(cache.ref, t_begin, t_end)


def refit_gram(cache: Cache, t_begin: int, t_end: int, gram, ws, per_head=True, stream=None):
    _check(lib().sks_refit_gram(cache.ref, t_begin, t_end, int(per_head), ptr(gram), ptr(ws),
                                _nbytes(ws), _stream(stream)))


def refit_basis(gram, basis, ws, eigval=None, stream=None):
    _check(lib().sks_refit_basis(ptr(gram), gram.shape[0], ptr(basis), ptr(eigval), ptr(ws),
                                 _nbytes(ws), _stream(stream)))


def refit_key_scale(cache: Cache, t_begin: int, t_end: int, basis, key_scale, ws,
                    basis_per_head=True, stream=None):
    _check(lib().sks_refit_key_scale(cache.ref, t_begin, t_end, ptr(basis), int(basis_per_head),
                                     ptr(key_scale), ptr(ws), _nbytes(ws), _stream(stream)))

