"""The frozen sketch basis in one file.

"8 agents x 250K context, concurrently, on two 3090s", "What it took": the
method ships a frozen sketch basis stored in one file, plus the script that
refits it (``python -m long_context_sparse_sketch_amd.refit``).  This module
reads and writes that file.  The pages give no format; this one is a plain
array file that C code can read without any library:

    offset  size                      field (little-endian)
    0       8                         magic  b"SKSBASIS"
    8       4                         int32  version (1)
    12      4                         int32  basis_per_head (0: one basis for all
                                             KV heads, 1: one per KV head)
    16      4                         int32  Hkv (KV heads; key scales stored)
    20      4                         int32  rank (64)
    24      4                         int32  D (head dim, 128)
    28      36                        zero
    64      4 * n * rank * D          float32 basis [n][rank][D], n = Hkv if
                                      basis_per_head else 1; row c of basis h
                                      is the c-th sketch direction of KV head h
    ...     4 * Hkv                   float32 key_scale [Hkv] (> 0)

The arrays are exactly the ``basis``, ``basis_per_head`` and ``key_scale``
arguments of sks_sketch_build, sks_sketch_build_query and sks_decode_step.
"""
from __future__ import annotations

import os
import struct

import numpy as np

MAGIC = b"SKSBASIS"
VERSION = 1
HEADER_BYTES = 64
_HEAD = struct.Struct("<8s5i")


class BasisFileError(ValueError):
    pass


def _n_basis(per_head: bool, Hkv: int) -> int:
    return Hkv if per_head else 1


def save(path: str, basis, key_scale, basis_per_head: bool | None = None) -> None:
    """Write `basis` ([rank][D], [1][rank][D] or [Hkv][rank][D] float32) and
    `key_scale` ([Hkv] float32, every value > 0) to `path`, atomically (the
    file is written next to `path` and renamed over it)."""
    b = np.ascontiguousarray(np.asarray(basis, dtype=np.float32))
    ks = np.ascontiguousarray(np.asarray(key_scale, dtype=np.float32).reshape(-1))
    if b.ndim == 2:
        b = b[None]
    if b.ndim != 3:
        raise BasisFileError(f"basis must be [rank][D] or [n][rank][D], got shape {b.shape}")
    Hkv = ks.shape[0]
    if basis_per_head is None:          # one basis per head when several are given
        basis_per_head = b.shape[0] > 1
    if b.shape[0] != _n_basis(basis_per_head, Hkv):
        raise BasisFileError(f"{b.shape[0]} bases for {Hkv} KV heads "
                             f"(basis_per_head={bool(basis_per_head)})")
    if Hkv < 1 or not np.all(np.isfinite(ks)) or not np.all(ks > 0):
        raise BasisFileError("key scales must be finite and > 0")
    if not np.all(np.isfinite(b)):
        raise BasisFileError("basis values must be finite")
    head = _HEAD.pack(MAGIC, VERSION, int(bool(basis_per_head)), Hkv, b.shape[1], b.shape[2])
    head += b"\0" * (HEADER_BYTES - len(head))
    tmp = f"{path}.tmp{os.getpid()}"
    with open(tmp, "wb") as f:
        f.write(head)
        f.write(b.astype("<f4").tobytes())
        f.write(ks.astype("<f4").tobytes())
    os.replace(tmp, path)


def load(path: str):
    """Read a basis file.  Returns (basis [n][rank][D] float32, key_scale
    [Hkv] float32, basis_per_head bool); raises BasisFileError on anything
    that is not a well-formed file of this format."""
    with open(path, "rb") as f:
        raw = f.read()
    if len(raw) < HEADER_BYTES:
        raise BasisFileError(f"{path}: {len(raw)} bytes, shorter than the {HEADER_BYTES}-byte header")
    magic, version, per_head, Hkv, rank, D = _HEAD.unpack_from(raw, 0)
    if magic != MAGIC:
        raise BasisFileError(f"{path}: not a sketch basis file (magic {magic!r})")
    if version != VERSION:
        raise BasisFileError(f"{path}: version {version}, expected {VERSION}")
    if per_head not in (0, 1) or Hkv < 1 or rank < 1 or D < 1:
        raise BasisFileError(f"{path}: bad header (per_head={per_head}, Hkv={Hkv}, "
                             f"rank={rank}, D={D})")
    if any(raw[_HEAD.size:HEADER_BYTES]):
        raise BasisFileError(f"{path}: reserved header bytes are not zero")
    n = _n_basis(bool(per_head), Hkv)
    want = HEADER_BYTES + 4 * (n * rank * D + Hkv)
    if len(raw) != want:
        raise BasisFileError(f"{path}: {len(raw)} bytes, the header implies {want}")
    body = np.frombuffer(raw, dtype="<f4", offset=HEADER_BYTES)
    basis = body[: n * rank * D].reshape(n, rank, D).astype(np.float32)
    ks = body[n * rank * D:].astype(np.float32)
    if not np.all(np.isfinite(basis)) or not np.all(np.isfinite(ks)) or not np.all(ks > 0):
        raise BasisFileError(f"{path}: non-finite values or key scales <= 0")
    return basis, ks, bool(per_head)
