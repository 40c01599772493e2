"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every entry point include/sks.h declares, sizes workspaces, and rejects
invalid arguments with an error code and text before launching anything.
Only argument combinations that fail validation are called here."""
import ctypes
import os
import re

import pytest

from long_context_sparse_sketch_amd import binding as sks
from long_context_sparse_sketch_amd import configs as C

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sks.h")
FAKE = 0x100000            # a non-NULL, aligned address: never dereferenced on failure paths


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(sks.LIB_PATH):
        from long_context_sparse_sketch_amd.build import build
        build()
    return sks.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sks_[a-z_]+)\s*\(", text)))


def test_header_declares_the_five_calls():
    names = declared_functions()
    for n in ("sks_sketch_build", "sks_sketch_score", "sks_topk_select", "sks_gather_pack",
              "sks_sparse_decode_attn"):
        assert n in names


def test_library_exports_every_declared_symbol(L):
    names = declared_functions()
    assert names and set(names) == set(sks.EXPORTS)
    for n in names:
        assert hasattr(L, n), n


def kv(B=2, Hkv=4, D=128, T=1000, dtype=sks.KV_BF16, K=FAKE, V=FAKE, Ks=0, Vs=0, sl=FAKE):
    return sks.KVDesc(B, Hkv, D, T, dtype, K, V, Ks or None, Vs or None, sl)


def call_attn(L, k, p, Hq=8, ws_bytes=1 << 30, q=FAKE, out=FAKE, idx=FAKE, ws=FAKE):
    return L.sks_sparse_decode_attn(q, Hq, ctypes.byref(k), ctypes.byref(p), idx, None, None,
                                    ctypes.c_float(0.088), out, None, ws, ws_bytes, None)


@pytest.mark.parametrize("mut,code,word", [
    (dict(D=64), sks.SKS_ERR_ARG, "D must be"),
    (dict(B=0), sks.SKS_ERR_ARG, "B and Hkv"),
    (dict(K=0), sks.SKS_ERR_ARG, "kv->K"),
    (dict(K=FAKE + 4), sks.SKS_ERR_ARG, "aligned"),
    (dict(sl=0), sks.SKS_ERR_ARG, "seq_len"),
    (dict(dtype=7), sks.SKS_ERR_ARG, "dtype"),
    (dict(dtype=sks.KV_I8), sks.SKS_ERR_ARG, "K_scale"),
    (dict(dtype=sks.KV_I4), sks.SKS_ERR_ARG, "K_scale"),
    (dict(dtype=sks.KV_I4, Ks=FAKE), sks.SKS_ERR_ARG, "V_scale"),
    (dict(B=8192, Hkv=8), sks.SKS_ERR_ARG, "65535"),     # segments: a grid dimension
])
def test_cache_description_errors(L, mut, code, word):
    k = kv(**mut)
    rc = call_attn(L, k, sks.params(64, 32))
    assert rc == code
    assert word in sks.last_error()


@pytest.mark.parametrize("p,Hq,word", [
    (sks.params(64, 32, rank=32), 8, "rank"),
    (sks.params(64, 0), 8, "topk"),
    (sks.params(64, (1 << 24) + 1), 8, "topk"),
    (sks.params(-1, 32), 8, "window"),
    (sks.params((1 << 24) + 1, 32), 8, "window"),
    (sks.params(64, 32, pool=0), 8, "pool"),
    (sks.params(64, 32, pool=65), 8, "pool"),
    (sks.params(64, 32, rows=9), 8, "rows"),
    (sks.params(64, 32), 6, "multiple"),
    (sks.params(64, 32), 4 * 9, "<= 8"),
])
def test_parameter_errors(L, p, Hq, word):
    assert call_attn(L, kv(), p, Hq=Hq) == sks.SKS_ERR_ARG
    assert word in sks.last_error()


def test_workspace_errors(L):
    rc = call_attn(L, kv(), sks.params(64, 32), ws_bytes=16)
    assert rc == sks.SKS_ERR_WORKSPACE and "workspace" in sks.last_error()
    rc = call_attn(L, kv(), sks.params(64, 32), ws=0)
    assert rc == sks.SKS_ERR_WORKSPACE


def hot(k, K_hot=FAKE, V_hot=FAKE, Ks=0, Vs=0, W=200):
    k.K_hot, k.V_hot = K_hot or None, V_hot or None
    k.K_hot_scale, k.V_hot_scale = Ks or None, Vs or None
    k.W_hot = W
    return k


@pytest.mark.parametrize("mut,p,code,word", [
    (dict(V_hot=0), sks.params(64, 32), sks.SKS_ERR_ARG, "both"),
    (dict(K_hot=0), sks.params(64, 32), sks.SKS_ERR_ARG, "both"),
    (dict(W=64), sks.params(64, 32), sks.SKS_ERR_ARG, "W_hot"),
    (dict(W=64), sks.params(63, 32, rows=2), sks.SKS_ERR_ARG, "W_hot"),   # window + rows > W_hot
    (dict(W=1001), sks.params(64, 32), sks.SKS_ERR_ARG, "W_hot"),    # > T_max
    (dict(K_hot=FAKE + 8), sks.params(64, 32), sks.SKS_ERR_ARG, "aligned"),
    (dict(), sks.params(64, 32, pool=4), sks.SKS_ERR_UNSUPPORTED, "pool"),
])
def test_hot_tier_errors(L, mut, p, code, word):
    k = hot(kv(), **mut)
    assert call_attn(L, k, p) == code
    assert word in sks.last_error()


def test_hot_tier_scales_required_for_codes(L):
    k = hot(kv(dtype=sks.KV_I4, Ks=FAKE, Vs=FAKE))
    assert call_attn(L, k, sks.params(64, 32)) == sks.SKS_ERR_ARG
    assert "K_hot_scale" in sks.last_error()
    k = hot(kv(dtype=sks.KV_I8, Ks=FAKE, Vs=FAKE), Ks=FAKE)
    assert call_attn(L, k, sks.params(64, 32)) == sks.SKS_ERR_ARG
    assert "V_hot_scale" in sks.last_error()


@pytest.mark.parametrize("dtype", [sks.KV_I8, sks.KV_I4])
def test_unsupported_code_cache_pooling(L, dtype):
    k = kv(dtype=dtype, Ks=FAKE, Vs=FAKE)
    rc = call_attn(L, k, sks.params(64, 32, pool=4))
    assert rc == sks.SKS_ERR_UNSUPPORTED


def test_sketch_build_argument_errors(L):
    k = kv()
    p = sks.params(64, 32)
    rc = L.sks_sketch_build(ctypes.byref(k), ctypes.byref(p), FAKE, 0, FAKE, 5, 2, FAKE, None,
                            None, None)
    assert rc == sks.SKS_ERR_ARG and "range" in sks.last_error()
    rc = L.sks_sketch_build(ctypes.byref(k), ctypes.byref(p), FAKE, 0, FAKE, 0, 10, FAKE, FAKE,
                            FAKE, None)
    assert rc == sks.SKS_ERR_ARG and "NULL when pool == 1" in sks.last_error()
    p4 = sks.params(64, 32, pool=4)
    rc = L.sks_sketch_build(ctypes.byref(k), ctypes.byref(p4), FAKE, 0, FAKE, 0, 10, FAKE, None,
                            None, None)
    assert rc == sks.SKS_ERR_ARG and "Kp" in sks.last_error()


def test_score_topk_query_gather_argument_errors(L):
    k, p = kv(), sks.params(64, 32)
    assert L.sks_sketch_score(None, FAKE, ctypes.byref(k), ctypes.byref(p), FAKE, None, 0,
                              None) == 1
    assert "qsk" in sks.last_error()
    assert L.sks_sketch_score(FAKE, FAKE, ctypes.byref(k), ctypes.byref(p), FAKE, FAKE, 8,
                              None) == sks.SKS_ERR_WORKSPACE
    assert L.sks_topk_select(FAKE, ctypes.byref(k), ctypes.byref(p), 0, FAKE, None, FAKE, 8,
                             None) == sks.SKS_ERR_WORKSPACE
    assert L.sks_topk_select(FAKE, ctypes.byref(k), ctypes.byref(p), 6, FAKE, None, FAKE,
                             1 << 30, None) == sks.SKS_ERR_ARG
    assert "flags" in sks.last_error()
    assert L.sks_workspace_init(None, 64, None) == sks.SKS_ERR_ARG
    assert L.sks_sketch_build_query(FAKE, 1, 1, 6, 4, FAKE, 0, FAKE, None, None) == 1
    assert "multiple" in sks.last_error()
    assert L.sks_gather_pack(ctypes.byref(k), ctypes.byref(p), FAKE, None, None, FAKE, FAKE,
                             FAKE, None, FAKE, None) == 1
    assert "NULL for bf16" in sks.last_error()


@pytest.mark.parametrize("cfg", C.ALL, ids=lambda c: c.name)
def test_workspace_sizes_cover_selection_and_attention(L, cfg):
    k = kv(B=cfg.B, Hkv=cfg.Hkv, T=cfg.T_max,
           dtype=sks.KV_I8 if cfg.kv_dtype == C.KV_I8 else sks.KV_BF16, Ks=FAKE, Vs=FAKE)
    if cfg.kv_dtype != C.KV_I8:
        k.K_scale = k.V_scale = None
    p = sks.params(cfg.window, cfg.topk, cfg.pool, cfg.R)
    nb = L.sks_workspace_bytes(ctypes.byref(k), ctypes.byref(p), cfg.Hq)
    nseg = cfg.B * cfg.R * cfg.Hkv
    NB = cfg.T_max // cfg.pool
    # histograms (zero at rest) + candidates (8 B per sketch row)
    assert nb >= nseg * 2048 * 4 + nseg * NB * 8
    # attention partials: at least one per 384 entries (the largest split)
    nsplit = -(-(cfg.topk + cfg.window + cfg.pool - 1) // 384)
    assert nb >= nseg * nsplit * cfg.g * (128 + 2) * 4
    assert L.sks_workspace_bytes(ctypes.byref(k), ctypes.byref(p), 0) == 0
    assert L.sks_workspace_bytes(ctypes.byref(k), ctypes.byref(p), 9 * cfg.Hkv) == 0


def expected_split(cfg):
    """128 entries for attention sets under 1,536, else 384 (bf16) or 256 (int8, int4)."""
    if cfg.topk + cfg.window + cfg.pool - 1 < 1536:
        return 128
    return 384 if cfg.kv_dtype == C.KV_BF16 else 256


SPLIT_CFGS = ([C.small(c) for c in C.ALL] + [C.full_set(c) for c in C.ALL[1:]] + list(C.ALL)
              + [C.with_kv(C.C3, C.KV_I4), C.with_kv(C.C3, C.KV_I8), C.with_kv(C.C1, C.KV_I4)])


def partial_splits(L, cfg, B, R):
    """Attention splits per segment, read off the workspace: only the partials,
    (m, l, acc[128]) fp32 per query head and split, grow with the group size."""
    quant = cfg.kv_dtype != C.KV_BF16
    k = kv(B=B, Hkv=cfg.Hkv, T=cfg.T_max, dtype=cfg.kv_dtype,
           Ks=FAKE if quant else None, Vs=FAKE if quant else None)
    p = sks.params(cfg.window, cfg.topk, cfg.pool, R)
    w1 = L.sks_workspace_bytes(ctypes.byref(k), ctypes.byref(p), cfg.Hkv)
    w2 = L.sks_workspace_bytes(ctypes.byref(k), ctypes.byref(p), 2 * cfg.Hkv)
    return round((w2 - w1) / (B * R * cfg.Hkv * (8 + 128 * 4)))


@pytest.mark.parametrize("cfg", SPLIT_CFGS, ids=lambda c: c.name)
def test_attention_split_follows_the_row_parameters(L, cfg):
    """The split is 128 entries for attention sets under 1,536, else 384 for
    bf16 rows and 256 for int8 / int4 rows; the same for any batch size and
    any number of verify rows (it fixes a row's order of operations)."""
    want = -(-(cfg.topk + cfg.window + cfg.pool - 1) // expected_split(cfg))
    assert partial_splits(L, cfg, cfg.B, cfg.R) == want
    for B, R in ((1, 1), (1, 8), (64, 1), (64, 3)):
        assert partial_splits(L, cfg, B, R) == want, (B, R)


MAX_ROWS = 8192 * 1024     # sketch rows (T_max / pool) the selection supports


@pytest.mark.parametrize("pool", [1, 4])
def test_cache_size_limit(L, pool):
    """T_max / pool above 8,388,608 is refused before any launch; at the limit
    the call gets as far as the workspace check."""
    p = sks.params(4096, 2048, pool)
    for T, code in ((MAX_ROWS * pool + pool, sks.SKS_ERR_UNSUPPORTED),
                    (MAX_ROWS * pool, sks.SKS_ERR_WORKSPACE)):
        k = kv(B=1, Hkv=1, T=T)
        rc = L.sks_topk_select(FAKE, ctypes.byref(k), ctypes.byref(p), 0, FAKE, None, FAKE, 8,
                               None)
        assert rc == code, (T, sks.last_error())
        if code == sks.SKS_ERR_UNSUPPORTED:
            assert "8388608" in sks.last_error()
        kw = dict(Kp=FAKE, Vp=FAKE) if pool > 1 else {}
        rc = L.sks_decode_step(ctypes.byref(k), ctypes.byref(p), ctypes.byref(step_desc(**kw)), 1,
                               FAKE, 8, None)
        assert rc == code, (T, sks.last_error())


def test_candidate_calls_argument_errors(L):
    k, p = kv(), sks.params(64, 32)
    sc = lambda flags=0, qsk=FAKE, S=FAKE, ws=FAKE, nb=1 << 30: L.sks_score_candidates(
        qsk, S, ctypes.byref(k), ctypes.byref(p), flags, ws, nb, None)
    assert sc(flags=8) == sks.SKS_ERR_ARG and "flags" in sks.last_error()
    assert sc(flags=sks.CAND_TEST_HIGH | sks.CAND_TEST_ZERO) == sks.SKS_ERR_ARG
    assert "exclude" in sks.last_error()
    assert sc(qsk=None) == sks.SKS_ERR_ARG and "qsk" in sks.last_error()
    assert sc(S=FAKE + 4) == sks.SKS_ERR_ARG and "aligned" in sks.last_error()
    assert sc(ws=None) == sks.SKS_ERR_WORKSPACE
    assert sc(nb=16) == sks.SKS_ERR_WORKSPACE
    sel = lambda scores=FAKE, idx=FAKE, n_sel=None, nb=1 << 30: L.sks_topk_select_candidates(
        FAKE, FAKE, ctypes.byref(k), ctypes.byref(p), scores, idx, n_sel, FAKE, nb, None)
    assert sel(scores=None) == sks.SKS_ERR_ARG and "scores" in sks.last_error()
    assert sel(idx=None) == sks.SKS_ERR_ARG and "idx" in sks.last_error()
    assert sel(n_sel=FAKE + 2) == sks.SKS_ERR_ARG and "n_sel" in sks.last_error()
    assert sel(nb=16) == sks.SKS_ERR_WORKSPACE


def step_desc(**kw):
    d = dict(q=FAKE, Hq=8, basis=FAKE, basis_per_head=0, key_scale=FAKE, S=FAKE, Kp=None, Vp=None,
             sm_scale=0.088, qsk=FAKE, qscale=None, scores=FAKE, idx=FAKE, n_sel=None, out=FAKE,
             lse=None)
    d.update(kw)
    return sks.StepDesc(*[d[f] for f, _ in sks.StepDesc._fields_])


def test_decode_step_argument_errors(L):
    k, p = kv(), sks.params(64, 32)
    call = lambda st, flags=1, ws=FAKE, nb=1 << 30: L.sks_decode_step(
        ctypes.byref(k), ctypes.byref(p), st if st is None else ctypes.byref(st), flags, ws, nb,
        None)
    assert call(None) == sks.SKS_ERR_ARG and "step" in sks.last_error()
    assert call(step_desc(), flags=16) == sks.SKS_ERR_ARG and "flags" in sks.last_error()
    assert call(step_desc(), flags=8 | 3) == sks.SKS_ERR_ARG and "flags" in sks.last_error()
    assert call(step_desc(Hq=6)) == sks.SKS_ERR_ARG and "multiple" in sks.last_error()
    assert call(step_desc(scores=None)) == sks.SKS_ERR_ARG and "scores" in sks.last_error()
    assert call(step_desc(out=FAKE + 4)) == sks.SKS_ERR_ARG and "aligned" in sks.last_error()
    assert call(step_desc(Kp=FAKE, Vp=FAKE)) == sks.SKS_ERR_ARG
    assert call(step_desc(sm_scale=0.0)) == sks.SKS_ERR_ARG and "sm_scale" in sks.last_error()
    assert call(step_desc(), nb=64) == sks.SKS_ERR_WORKSPACE
    p4 = sks.params(64, 32, pool=4)
    assert L.sks_decode_step(ctypes.byref(k), ctypes.byref(p4), ctypes.byref(step_desc()), 1,
                             FAKE, 1 << 30, None) == sks.SKS_ERR_ARG
    assert "Kp" in sks.last_error()


def test_workspace_holds_selection_and_attention_scratch_apart(L):
    """The selection scratch and the attention partials are separate regions:
    the workspace holds their sum (partials: at least one per 384 entries)."""
    k, p = kv(B=8, Hkv=4, T=250000), sks.params(4096, 2048)
    small = L.sks_workspace_bytes(ctypes.byref(k), ctypes.byref(p), 24)
    n_sub = -(-250000 // 1024)
    cand = 32 * n_sub * 1024 * 8
    part = 32 * (-(-2048 // 384) + -(-4096 // 384)) * 6 * (8 + 512)
    assert small >= cand + part


def test_refit_argument_errors(L):
    k = kv(T=1000)
    assert L.sks_refit_workspace_bytes(ctypes.byref(k), 0, 1000) > 0
    assert L.sks_refit_workspace_bytes(ctypes.byref(k), 0, 1001) == 0
    assert "key range" in sks.last_error()
    assert L.sks_refit_workspace_bytes(ctypes.byref(k), 5, 4) == 0
    assert L.sks_refit_gram(ctypes.byref(k), 0, 1000, 1, FAKE, FAKE, 16, None) == \
        sks.SKS_ERR_WORKSPACE
    assert L.sks_refit_gram(ctypes.byref(k), 0, 1000, 1, FAKE + 4, FAKE, 1 << 30, None) == \
        sks.SKS_ERR_ARG and "aligned" in sks.last_error()
    k8 = kv(T=1000, dtype=sks.KV_I8, Ks=FAKE, Vs=FAKE)
    assert L.sks_refit_gram(ctypes.byref(k8), 0, 10, 1, FAKE, FAKE, 1 << 30, None) == \
        sks.SKS_ERR_UNSUPPORTED and "bf16" in sks.last_error()
    assert L.sks_refit_basis(FAKE, 0, FAKE, None, FAKE, 1 << 30, None) == sks.SKS_ERR_ARG
    assert L.sks_refit_basis(FAKE, 2, FAKE, None, FAKE, 128 * 128 * 8, None) == \
        sks.SKS_ERR_WORKSPACE
    assert L.sks_refit_key_scale(ctypes.byref(k), 0, 1000, None, 1, FAKE, FAKE, 1 << 30,
                                 None) == sks.SKS_ERR_ARG and "basis" in sks.last_error()


def test_static_step_argument_errors_and_size_limit(L):
    """The allocation-free step validates like sks_decode_step, before any
    launch, and refuses shapes whose workspace exceeds its static array."""
    k, p = kv(), sks.params(64, 32)
    call = lambda st, flags=1, kk=k, pp=p: L.sks_decode_step_static(
        ctypes.byref(kk), ctypes.byref(pp), st if st is None else ctypes.byref(st), flags, None)
    assert call(None) == sks.SKS_ERR_ARG and "step" in sks.last_error()
    assert call(step_desc(), flags=16) == sks.SKS_ERR_ARG and "flags" in sks.last_error()
    assert call(step_desc(Hq=6)) == sks.SKS_ERR_ARG and "multiple" in sks.last_error()
    assert call(step_desc(idx=None)) == sks.SKS_ERR_ARG and "idx" in sks.last_error()
    # a shape beyond the static workspace: refused with the sizes in the message
    big = kv(B=64, Hkv=8, T=250000)
    need = L.sks_workspace_bytes(ctypes.byref(big), ctypes.byref(p), 8)
    assert need > sks.STATIC_WORKSPACE_BYTES
    assert call(step_desc(), kk=big) == sks.SKS_ERR_WORKSPACE
    assert str(need) in sks.last_error() and str(sks.STATIC_WORKSPACE_BYTES) in sks.last_error()


def test_static_workspace_size_matches_header_and_fits_every_workload(L):
    text = open(HEADER).read()
    m = re.search(r"#define SKS_STATIC_WORKSPACE_BYTES \((\d+)u << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == sks.STATIC_WORKSPACE_BYTES
    from long_context_sparse_sketch_amd import configs as C
    for cfg in C.ALL:
        k = kv(B=cfg.B, Hkv=cfg.Hkv, T=cfg.T_max, dtype=cfg.kv_dtype, Ks=FAKE, Vs=FAKE)
        p = sks.params(cfg.window, cfg.topk, cfg.pool, cfg.R)
        need = L.sks_workspace_bytes(ctypes.byref(k), ctypes.byref(p), cfg.Hq)
        assert 0 < need <= sks.STATIC_WORKSPACE_BYTES, (cfg.name, need)
