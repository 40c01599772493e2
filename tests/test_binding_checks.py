"""The Python binding checks every tensor against the layout sks.h gives it
(contiguous, exact byte size for the cache and parameters, on the GPU) before
calling the library, so a wrongly sized buffer raises instead of reaching a
kernel.  CPU only: every case here raises before any call into libsks."""
import ctypes

import pytest
import torch

from long_context_sparse_sketch_amd import binding as sks

B, HKV, T, W, K_SEL, R, HQ = 2, 2, 1000, 64, 32, 3, 8


def cache(dtype=sks.KV_BF16):
    """A cache descriptor as Cache builds it (its tensors are never touched)."""
    c = sks.Cache.__new__(sks.Cache)
    c.desc = sks.KVDesc(B, HKV, 128, T, dtype, 16, 16, 16 if dtype else None,
                        16 if dtype else None, 16, None, None, None, None, 0)
    return c


P = sks.params(W, K_SEL, 1, R)


def t(*shape, dtype=torch.int32):
    return torch.zeros(shape, dtype=dtype)


def good():
    """Correctly sized (host) tensors of a step."""
    return dict(q=t(B, R, HQ, 128, dtype=torch.bfloat16), basis=t(1, 64, 128, dtype=torch.float32),
                key_scale=t(HKV, dtype=torch.float32), S=t(B, HKV, T, 64, dtype=torch.int8),
                qsk=t(B, R, HKV, 64, dtype=torch.int8), scores=t(B, R, HKV, T),
                idx=t(B, R, HKV, K_SEL), out=t(B, R, HQ, 128, dtype=torch.float32),
                ws=t(4096, dtype=torch.uint8))


def step(**kw):
    a = good()
    a.update(kw)
    sks.decode_step(cache(), P, a["q"], a["basis"], a["key_scale"], a["S"], a["qsk"], a["scores"],
                    a["idx"], a["out"], a["ws"])


@pytest.mark.parametrize("name,bad", [
    ("scores", t(B, R, HKV, T - 1)),
    ("idx", t(B, R, HKV, K_SEL + 1)),
    ("out", t(B, R, HQ, 128, dtype=torch.bfloat16)),
    ("S", t(B, HKV, T, 32, dtype=torch.int8)),
    ("qsk", t(B, 1, HKV, 64, dtype=torch.int8)),
    ("basis", t(2, 64, 128, dtype=torch.float32)),     # per-KV-head size, shared basis asked for
    ("key_scale", t(HKV + 1, dtype=torch.float32)),
])
def test_wrong_size_raises_before_the_call(name, bad):
    with pytest.raises(ValueError, match=f"^{name}: .* bytes expected"):
        step(**{name: bad})


def test_layout_of_q_checked():
    with pytest.raises(ValueError, match="q must be"):
        step(q=t(B, R, HQ, 64, dtype=torch.bfloat16))


def test_non_contiguous_raises():
    with pytest.raises(ValueError, match="scores must be contiguous"):
        step(scores=t(B, R, HKV, 2 * T)[..., ::2])


def test_host_tensor_of_the_right_size_must_be_on_the_gpu():
    with pytest.raises(ValueError, match="must be a GPU tensor"):
        step()


def test_individual_calls_check_sizes():
    c, a = cache(), good()
    with pytest.raises(ValueError, match="^scores: "):
        sks.sketch_score(a["qsk"], a["S"], c, P, t(B, R, HKV, T + 1), None)
    with pytest.raises(ValueError, match="^n_sel: "):
        sks.topk_select(a["scores"], c, P, a["idx"], t(B, R), a["ws"])
    with pytest.raises(ValueError, match="^lse: "):
        sks.sparse_decode_attn(a["q"], c, P, a["idx"], a["out"], a["ws"],
                               lse=t(B, R, HQ + 1, dtype=torch.float32))
    C = K_SEL + W
    with pytest.raises(ValueError, match="^K_out: "):
        sks.gather_pack(c, P, a["idx"], t(B, R, HKV, C, 64, dtype=torch.bfloat16),
                        t(B, R, HKV, C, 128, dtype=torch.bfloat16), t(B, R, HKV))
    with pytest.raises(ValueError, match="^Ks_out: "):
        sks.gather_pack(cache(sks.KV_I8), P, a["idx"], t(B, R, HKV, C, 128, dtype=torch.int8),
                        t(B, R, HKV, C, 128, dtype=torch.int8), t(B, R, HKV),
                        Ks_out=t(B, R, HKV, C - 1, dtype=torch.int16))
    with pytest.raises(ValueError, match="^qscale: "):
        sks.sketch_build_query(a["q"], HKV, a["basis"], a["qsk"], qscale=t(B, R, dtype=torch.float32))
    with pytest.raises(ValueError, match="^Kp: "):
        sks.sketch_build(c, sks.params(W, K_SEL, 4, R), a["basis"], a["key_scale"],
                         t(B, HKV, T // 4, 64, dtype=torch.int8),
                         Kp=t(B, HKV, T, 128, dtype=torch.bfloat16),
                         Vp=t(B, HKV, T // 4, 128, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="gram must be"):
        sks.refit_basis(t(128, 128, dtype=torch.float64), t(1, 64, 128, dtype=torch.float32),
                        a["ws"])
    with pytest.raises(ValueError, match="^eigval: "):
        sks.refit_basis(t(2, 128, 128, dtype=torch.float64), t(2, 64, 128, dtype=torch.float32),
                        a["ws"], eigval=t(1, 128, dtype=torch.float64))


def test_cache_checks():
    K = t(B, HKV, T, 128, dtype=torch.bfloat16)
    sl = t(B)
    with pytest.raises(ValueError, match="K must be \\[B\\]"):
        sks.Cache(t(B, T, 128, dtype=torch.bfloat16), K, sl)
    with pytest.raises(ValueError, match="bfloat16, int8 or uint8"):
        sks.Cache(t(B, HKV, T, 128, dtype=torch.float32), K, sl)
    with pytest.raises(ValueError, match="must have K's dtype"):
        sks.Cache(K, t(B, HKV, T, 128, dtype=torch.int8), sl)
    K8 = t(B, HKV, T, 128, dtype=torch.int8)
    with pytest.raises(ValueError, match="need K_scale and V_scale"):
        sks.Cache(K8, K8, sl)
    with pytest.raises(ValueError, match="^V: "):
        sks.Cache(K, t(B, HKV, T - 1, 128, dtype=torch.bfloat16), sl)
    with pytest.raises(ValueError, match="pinned"):
        sks.Cache(K, K, sl)                      # host memory that is not pinned


def test_checks_do_not_reach_the_library():
    # the last error text of the library is untouched by the binding's checks
    L = sks.lib()
    L.sks_workspace_bytes(None, None, 0)
    before = sks.last_error()
    with pytest.raises(ValueError):
        step(out=t(1))
    assert sks.last_error() == before
    assert ctypes.c_size_t(L.sks_workspace_bytes(None, None, 0)).value == 0
