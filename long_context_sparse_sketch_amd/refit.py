"""Refit the sketch basis from captured keys and freeze it in one file.

"8 agents x 250K context, concurrently, on two 3090s", "What it took": a
frozen sketch basis (one file) plus the script to refit it.

    python -m long_context_sparse_sketch_amd.refit --keys keys.npy --out basis.sksb
    python -m long_context_sparse_sketch_amd.refit --synthetic 2,4,20000 --out basis.sksb

``--keys`` takes captured keys as a ``.npy`` array of bfloat16 bit patterns
``[B][Hkv][T][128]`` (uint16; ``--lengths`` optionally gives the captured
length of each sequence, ``[B]`` int32); ``--synthetic B,Hkv,T`` draws the
seeded planted-spectrum stand-in keys (no model keys ship with this code).
The refit runs on the GPU through the C ABI (sks_refit_gram,
sks_refit_basis, sks_refit_key_scale: the principal directions of the keys
and the clip-free key scale) and the result is written with basis_file.save.
"""
from __future__ import annotations

import argparse
import sys

import numpy as np
import torch

from . import basis_file
from . import binding as sks


def refit(cache: sks.Cache, t_begin: int, t_end: int, per_head: bool = True, stream=None):
    """Refit on the keys [t_begin, min(t_end, seq_len[b])) of every sequence of
    `cache` (bf16).  Returns device tensors (basis [n][64][128] float32,
    key_scale [Hkv] float32, eigenvalues [n][128] float64), n = Hkv or 1."""
    dev = cache.seq_len.device
    nb = sks.refit_workspace_bytes(cache, t_begin, t_end)
    if nb == 0:
        raise sks.SksError(sks.SKS_ERR_ARG, sks.last_error())
    Hkv = cache.desc.Hkv
    n = Hkv if per_head else 1
    ws = torch.empty(nb, dtype=torch.uint8, device=dev)
    gram = torch.empty((n, sks.HEAD_DIM, sks.HEAD_DIM), dtype=torch.float64, device=dev)
    basis = torch.empty((n, sks.RANK, sks.HEAD_DIM), dtype=torch.float32, device=dev)
    eig = torch.empty((n, sks.HEAD_DIM), dtype=torch.float64, device=dev)
    key_scale = torch.empty(Hkv, dtype=torch.float32, device=dev)
    sks.refit_gram(cache, t_begin, t_end, gram, ws, per_head=per_head, stream=stream)
    sks.refit_basis(gram, basis, ws, eigval=eig, stream=stream)
    sks.refit_key_scale(cache, t_begin, t_end, basis, key_scale, ws, basis_per_head=per_head,
                        stream=stream)
    return basis, key_scale, eig


def refit_to_file(cache: sks.Cache, t_begin: int, t_end: int, path: str,
                  per_head: bool = True):
    """Refit (see `refit`) and write the frozen basis file; returns the host
    arrays written (basis [n][64][128], key_scale [Hkv])."""
    basis, key_scale, _ = refit(cache, t_begin, t_end, per_head)
    torch.cuda.synchronize()
    b, ks = basis.cpu().numpy(), key_scale.cpu().numpy()
    basis_file.save(path, b, ks, basis_per_head=per_head)
    return b, ks


def _keys_cache(K_bits: np.ndarray, lengths: np.ndarray | None, device) -> sks.Cache:
    if K_bits.dtype != np.uint16 or K_bits.ndim != 4 or K_bits.shape[3] != sks.HEAD_DIM:
        raise ValueError(f"keys must be uint16 bf16 bits [B][Hkv][T][{sks.HEAD_DIM}], "
                         f"got {K_bits.dtype} {K_bits.shape}")
    B, _, T, _ = K_bits.shape
    L = np.full(B, T, np.int32) if lengths is None else np.asarray(lengths, np.int32).reshape(B)
    K = torch.from_numpy(np.ascontiguousarray(K_bits).view(np.int16)).to(device).view(torch.bfloat16)
    sl = torch.from_numpy(L.copy()).to(device)
    return sks.Cache(K, K, sl)


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    src = ap.add_mutually_exclusive_group(required=True)
    src.add_argument("--keys", help="captured keys: .npy of bf16 bits [B][Hkv][T][128] uint16")
    src.add_argument("--synthetic", help="B,Hkv,T: seeded planted-spectrum stand-in keys")
    ap.add_argument("--lengths", help=".npy [B] int32: captured length of each sequence")
    ap.add_argument("--seed", type=int, default=1)
    ap.add_argument("--t-begin", type=int, default=0)
    ap.add_argument("--t-end", type=int, default=None)
    ap.add_argument("--shared", action="store_true", help="one basis for all KV heads")
    ap.add_argument("--out", required=True, help="basis file to write")
    args = ap.parse_args(argv)
    if not torch.cuda.is_available():
        print("refit: a GPU is required (the refit runs in the HIP kernels)", file=sys.stderr)
        return 2
    if args.keys:
        K = np.load(args.keys, allow_pickle=False)
        lengths = np.load(args.lengths, allow_pickle=False) if args.lengths else None
    else:
        from .synth import make_refit_keys
        B, Hkv, T = (int(x) for x in args.synthetic.split(","))
        K, _, _ = make_refit_keys(B, Hkv, T, seed=args.seed)
        lengths = None
    cache = _keys_cache(K, lengths, "cuda")
    t_end = K.shape[2] if args.t_end is None else args.t_end
    b, ks = refit_to_file(cache, args.t_begin, t_end, args.out, per_head=not args.shared)
    print(f"refit: {b.shape[0]} basis(es) of {b.shape[1]}x{b.shape[2]}, key scales "
          f"{np.array2string(ks, precision=5)} -> {args.out}")
    return 0


if __name__ == "__main__":
    sys.exit(main())
