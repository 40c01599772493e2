"""GPU parity of the sketch-basis refit ("8 agents x 250K context ...",
"What it took": a frozen sketch basis plus the script to refit it) against the
oracle, through the C ABI.

Bars, derived from the arithmetic:
* Gram matrix: each wave sums exact bf16 products over at most 2,048 keys in
  fp32 and four waves are added in fp32, so |G_gpu - G| <= (2048 + 3) u
  sqrt(G_ii G_jj) with u = 2^-24 (Cauchy-Schwarz bounds the sum of |x_i x_j|);
  the chunks are added in fp64.  Tolerance 2e-4 sqrt(G_ii G_jj).
* basis, given the oracle's Gram matrix: fp64 Jacobi against LAPACK in fp64;
  the eigenvectors are well separated here, so both agree far below the fp32
  rounding of the output: |basis_gpu - fp32(basis)| <= 1e-6, eigenvalues to
  1e-10 of the largest.
* key scale, given the basis: 128 exact products summed in fp32, |y| within
  128 u of exact: relative 2e-5.
"""
import numpy as np
import pytest
import torch

from long_context_sparse_sketch_amd import binding as sks
from long_context_sparse_sketch_amd import configs as C
from long_context_sparse_sketch_amd.runtime import to_device
from long_context_sparse_sketch_amd.synth import distinct_diagonal, make_case, make_refit_keys
from oracle import sks_oracle as orc
from tests.gpu_util import flush

pytestmark = pytest.mark.gpu


def gpu_refit(K_bits, seq_len, t_begin, t_end, per_head=True, basis_in=None, gram_in=None):
    """Run the three refit calls; returns numpy (gram, basis, eigval, key_scale).
    basis_in / gram_in replace the GPU's own intermediate (oracle values)."""
    B, Hkv, T, _ = K_bits.shape
    K = to_device(K_bits, bf16=True)
    sl = torch.from_numpy(np.asarray(seq_len, np.int32).copy()).cuda()
    cache = sks.Cache(K, K, sl)
    nb = sks.refit_workspace_bytes(cache, t_begin, t_end)
    assert nb > 0, sks.last_error()
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    nmat = Hkv if per_head else 1
    G = torch.empty((nmat, 128, 128), dtype=torch.float64, device="cuda")
    sks.refit_gram(cache, t_begin, t_end, G, ws, per_head=per_head)
    if gram_in is not None:
        G.copy_(torch.from_numpy(gram_in))
    basis = torch.empty((nmat, 64, 128), dtype=torch.float32, device="cuda")
    eig = torch.empty((nmat, 128), dtype=torch.float64, device="cuda")
    sks.refit_basis(G, basis, ws, eigval=eig)
    if basis_in is not None:
        basis.copy_(torch.from_numpy(basis_in.astype(np.float32)))
    scale = torch.empty(Hkv, dtype=torch.float32, device="cuda")
    sks.refit_key_scale(cache, t_begin, t_end, basis, scale, ws, basis_per_head=per_head)
    torch.cuda.synchronize()
    out = [t.cpu().numpy() for t in (G, basis, eig, scale)]
    if gram_in is not None:
        out[0] = None
    return out


def check_gram(G_gpu, G_ref):
    assert np.array_equal(G_gpu, np.swapaxes(G_gpu, 1, 2))            # exactly symmetric
    for m in range(G_ref.shape[0]):
        d = np.sqrt(np.outer(np.diag(G_ref[m]), np.diag(G_ref[m])))
        assert (np.abs(G_gpu[m] - G_ref[m]) <= 2e-4 * d + 1e-30).all(), m


def check_basis(basis_gpu, eig_gpu, G_ref):
    for m in range(G_ref.shape[0]):
        P, w = orc.basis_from_gram(G_ref[m])
        np.testing.assert_allclose(eig_gpu[m], w, rtol=0, atol=1e-10 * abs(w[0]))
        assert np.abs(basis_gpu[m] - P.astype(np.float32)).max() <= 1e-6, m


def check_scale(scale_gpu, K_bits, seq_len, t_begin, t_end, basis, per_head):
    for h in range(K_bits.shape[1]):
        keys = orc.refit_keys(K_bits, seq_len, h, t_begin, t_end)
        want = orc.refit_key_scale(keys, basis[h if per_head else 0].astype(np.float64))
        assert abs(scale_gpu[h] - want) <= 2e-5 * want, (h, scale_gpu[h], want)


@pytest.mark.parametrize("per_head", [True, False])
def test_refit_planted_keys(per_head):
    B, Hkv, T = 2, 3, 20000
    K, U, sigma = make_refit_keys(B, Hkv, T, seed=91)
    sl = np.array([20000, 13001], np.int32)                         # ragged lengths
    t0, t1 = 100, 19000                                              # several chunks + tails
    flush(f"[refit] planted {B}x{Hkv}x{T} per_head={per_head}")
    G_ref, P_ref, w_ref, s_ref = orc.refit(K, sl, t0, t1, per_head=per_head)
    G, basis, eig, scale = gpu_refit(K, sl, t0, t1, per_head)
    check_gram(G, G_ref)
    # each stage on the oracle's input
    _, basis2, eig2, _ = gpu_refit(K, sl, t0, t1, per_head, gram_in=G_ref)
    check_basis(basis2, eig2, G_ref)
    *_, scale3 = gpu_refit(K, sl, t0, t1, per_head, basis_in=P_ref)
    check_scale(scale3, K, sl, t0, t1, P_ref, per_head)
    # end to end: a per-head basis spans its head's planted subspace (a shared
    # one mixes the heads' differently rotated spectra), and no captured key's
    # code clips under the GPU's own scale
    if per_head:
        for h in range(Hkv):
            proj = basis[h].astype(np.float64).T @ basis[h].astype(np.float64)
            assert np.abs(proj - U[h][:, :64] @ U[h][:, :64].T).max() < 0.05
    for h in range(Hkv):
        keys = orc.refit_keys(K, sl, h, t0, t1)
        y = orc.project(keys, basis[h if per_head else 0].astype(np.float64))
        assert np.abs(y).max() <= 127 * float(scale[h]) * (1 + 1e-5)


def test_refit_diagonal_gram_and_degenerate_ranges():
    # a diagonal Gram matrix: the basis is the coordinate axes of its 64 largest entries
    d = distinct_diagonal(128, seed=3)
    G_in = np.diag(d)[None]
    K = np.zeros((1, 1, 64, 128), np.uint16)
    _, basis, eig, _ = gpu_refit(K, [64], 0, 64, gram_in=G_in)
    assert list(eig[0]) == sorted(d, reverse=True)
    for r in range(64):
        e = np.zeros(128, np.float32)
        e[int(np.argmax(d == 128 - r))] = 1.0
        assert np.array_equal(basis[0, r], e)
    # empty key range and all-zero keys: zero Gram, scale 1, no fault
    G, _, _, scale = gpu_refit(K, [64], 10, 10)
    assert not G.any() and scale[0] == 1.0
    G, _, _, scale = gpu_refit(K, [0], 0, 64)                          # length 0
    assert not G.any() and scale[0] == 1.0


def test_refit_full_size_key_range():
    """On the 8 x 250K benchmark cache (N(0,1) keys, 4 KV heads), over a
    60,000-position range of every sequence."""
    cfg = C.C3
    flush("[refit] generating the 8 x 250K cache")
    case = make_case(cfg)
    t0, t1 = 1000, 61000
    G_ref, P_ref, w_ref, s_ref = orc.refit(case.K, case.seq_len, t0, t1, per_head=True)
    G, basis, eig, scale = gpu_refit(case.K, case.seq_len, t0, t1)
    check_gram(G, G_ref)
    _, basis2, eig2, _ = gpu_refit(case.K, case.seq_len, t0, t1, gram_in=G_ref)
    check_basis(basis2, eig2, G_ref)
    *_, scale3 = gpu_refit(case.K, case.seq_len, t0, t1, basis_in=P_ref)
    check_scale(scale3, case.K, case.seq_len, t0, t1, P_ref, True)
