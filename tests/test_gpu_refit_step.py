"""The refit basis driving the step ("8 agents x 250K context ...", "What it
took": a frozen sketch basis in one file plus the script that refits it).

Captured keys (the planted-spectrum stand-in) are refitted on the GPU by the
refit script's code path, frozen in a basis file, read back, and used as a
per-KV-head basis with its refitted (non-power-of-two) key scales for the
bulk sketch build and the decode step.  Every stage is compared with the
oracle run on the same file contents:
* key and query codes within the sketch bound;
* scores and indices bit-exact on the oracle's codes, attention within
  tolerance on the oracle's indices;
* the whole step from the GPU's own codes: indices bit-exact against the
  oracle's selection on those codes, outputs within tolerance;
* candidate mode on the same codes selects the same indices.
"""
import numpy as np
import pytest
import torch

from long_context_sparse_sketch_amd import basis_file
from long_context_sparse_sketch_amd import binding as sks
from long_context_sparse_sketch_amd import refit as refit_script
from long_context_sparse_sketch_amd.runtime import SparseDecodeLayer, to_device
from long_context_sparse_sketch_amd.synth import f32_to_bf16_bits, make_refit_keys
from oracle import sks_oracle as orc
from tests.gpu_util import assert_attn_close, flush, lse_close, sketch_ok

pytestmark = pytest.mark.gpu


def test_refit_script_writes_a_loadable_file(tmp_path):
    out = str(tmp_path / "basis.sksb")
    assert refit_script.main(["--synthetic", "2,3,3000", "--seed", "5", "--out", out]) == 0
    basis, ks, per_head = basis_file.load(out)
    assert per_head and basis.shape == (3, 64, 128) and ks.shape == (3,)
    K, _, _ = make_refit_keys(2, 3, 3000, seed=5)
    for h in range(3):
        keys = orc.refit_keys(K, [3000, 3000], h, 0, 3000)
        y = orc.project(keys, basis[h].astype(np.float64))
        assert np.abs(y).max() <= 127 * float(ks[h]) * (1 + 1e-5)      # no captured key clips
        assert np.abs(y).max() >= 127 * float(ks[h]) * (1 - 1e-5)      # and the scale is tight
    out2 = str(tmp_path / "shared.sksb")
    assert refit_script.main(["--synthetic", "2,3,3000", "--seed", "5", "--shared",
                              "--out", out2]) == 0
    b2, ks2, ph2 = basis_file.load(out2)
    assert not ph2 and b2.shape == (1, 64, 128) and ks2.shape == (3,)


@pytest.mark.parametrize("R", [1, 3])
def test_refitted_basis_file_drives_the_step(tmp_path, R):
    B, Hkv, Hq, T = 2, 4, 24, 20011
    window, topk = 1000, 700
    g = Hq // Hkv
    flush(f"[refit-step] R={R}: keys {B}x{Hkv}x{T}")
    K, _, _ = make_refit_keys(B, Hkv, T, seed=77)
    rng = np.random.default_rng(78)
    V = f32_to_bf16_bits(rng.standard_normal((B, Hkv, T, 128)).astype(np.float32))
    q = f32_to_bf16_bits(rng.standard_normal((B, R, Hq, 128)).astype(np.float32))
    seq_len = np.array([T - R + 1, 15001], np.int32)          # ragged

    Kd, Vd = to_device(K, bf16=True), to_device(V, bf16=True)
    sl = torch.from_numpy(seq_len.copy()).cuda()
    cache = sks.Cache(Kd, Vd, sl)
    # refit on the captured keys [0, L_b), frozen in one file, read back
    path = str(tmp_path / "refit.sksb")
    refit_script.refit_to_file(cache, 0, T, path, per_head=True)
    basis, key_scale, per_head = basis_file.load(path)
    assert per_head and basis.shape == (Hkv, 64, 128)
    assert not np.any(np.log2(key_scale) == np.round(np.log2(key_scale))), key_scale
    # the file holds a refit of these keys: the oracle's basis spans the same
    # directions (loose: the GPU's Gram matrix sums in fp32), and the scales
    # leave no captured key clipped
    _, P_ref, _, s_ref = orc.refit(K, seq_len, 0, T, per_head=True)
    for h in range(Hkv):
        assert np.abs(basis[h] - P_ref[h]).max() < 1e-4, h
        assert abs(key_scale[h] - s_ref[h]) <= 2e-5 * s_ref[h], h

    layer = SparseDecodeLayer(B, R, Hq, Hkv, T, window, topk).bind(
        cache, torch.from_numpy(basis).cuda(), torch.from_numpy(key_scale).cuda(),
        basis_per_head=True)
    qd = to_device(q, bf16=True)
    layer.build_sketch(0, T)
    layer.step(qd)
    torch.cuda.synchronize()
    S_gpu, qsk_gpu = layer.S.cpu().numpy(), layer.qsk.cpu().numpy()
    flush(f"[refit-step] R={R}: oracle")
    ref = orc.decode_step(q, K, V, None, None, seq_len, basis, key_scale, window, topk, 1,
                          orc.KV_BF16)

    # 1. codes within the sketch bound, per head with its own basis and scale
    qf = orc.bf16_to_f64(q)
    for b in range(B):
        for h in range(Hkv):
            y = orc.project(orc.bf16_to_f64(K[b, h]), basis[h])
            assert sketch_ok(S_gpu[b, h], y, float(key_scale[h])).all(), (b, h)
            for i in range(R):
                _, s, yq = orc.query_sketch(qf[b, i, h * g:(h + 1) * g], basis[h])
                assert sketch_ok(qsk_gpu[b, i, h], yq, s).all(), (b, i, h)

    # 2. scores and indices bit-exact on the oracle's codes; attention on its indices
    kc = np.stack([np.stack([ref[(b, h)]["kcodes"] for h in range(Hkv)]) for b in range(B)])
    qc = np.zeros((B, R, Hkv, 64), np.int8)
    idx_ref = np.zeros((B, R, Hkv, topk), np.int32)
    for (b, h), r in ref.items():
        for i in range(R):
            qc[b, i, h] = r["qcode"][i]
            idx_ref[b, i, h] = r["idx"][i]
    kcd, qcd = torch.from_numpy(kc).cuda(), torch.from_numpy(qc).cuda()
    layer.score(qsk=qcd, S=kcd)
    layer.select()
    torch.cuda.synchronize()
    scores, idx = layer.scores.cpu().numpy(), layer.idx.cpu().numpy()
    for (b, h), r in ref.items():
        for i in range(R):
            n = len(r["scores"][i])
            assert np.array_equal(scores[b, i, h, :n], r["scores"][i]), (b, i, h)
            assert np.array_equal(idx[b, i, h], r["idx"][i]), (b, i, h)
    layer.attend(qd, idx=torch.from_numpy(idx_ref).cuda())
    torch.cuda.synchronize()
    out, lse = layer.out.cpu().numpy(), layer.lse.cpu().numpy()
    for (b, h), r in ref.items():
        for i in range(R):
            sl_ = slice(h * g, (h + 1) * g)
            assert_attn_close(out[b, i, sl_], r["out"][i], f"given idx {(b, i, h)}")
            lse_close(lse[b, i, sl_], r["lse"][i], f"given idx {(b, i, h)}")
    # candidate mode on the same codes: the same selection
    if R == 1:
        layer.score_candidates(qsk=qcd, S=kcd)
        layer.idx.fill_(-7)
        layer.select_candidates(qsk=qcd, S=kcd)
        torch.cuda.synchronize()
        assert np.array_equal(layer.idx.cpu().numpy(), idx_ref)

    # 3. the whole step from the GPU's own codes, against the oracle on them
    layer.build_sketch(0, T)
    layer.step(qd)
    torch.cuda.synchronize()
    own = orc.decode_step(q, K, V, None, None, seq_len, basis, key_scale, window, topk, 1,
                          orc.KV_BF16, codes=(layer.S.cpu().numpy(), layer.qsk.cpu().numpy()))
    idx, n_sel = layer.idx.cpu().numpy(), layer.n_sel.cpu().numpy()
    out, lse = layer.out.cpu().numpy(), layer.lse.cpu().numpy()
    for (b, h), r in own.items():
        for i in range(R):
            assert np.array_equal(idx[b, i, h], r["idx"][i]), ("own", b, i, h)
            assert n_sel[b, i, h] == r["n_sel"][i]
            sl_ = slice(h * g, (h + 1) * g)
            assert_attn_close(out[b, i, sl_], r["out"][i], f"own codes {(b, i, h)}")
            lse_close(lse[b, i, sl_], r["lse"][i], f"own codes {(b, i, h)}")
