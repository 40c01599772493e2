"""Host-RAM tier of the KV cache ("8 agents x 250K context, concurrently, on
two 3090s", claims list: the full cache in system RAM, the sketch and a small
hot set on the GPU, only the picked tokens across PCIe).

K/V live in pinned host memory that the kernels read through its device
address; the exact window and the rows' own tokens come from a ring of W_hot
slots in device memory.  The tier changes where rows are read, never what is
computed, so every output must equal the all-device run bit for bit.  To show
that window rows really come from the ring, the host copy of every position
that no row may read from host (each row's window and beyond) is poisoned,
and so is every ring slot that holds no valid position."""
import numpy as np
import pytest
import torch

from long_context_sparse_sketch_amd import binding as sks
from long_context_sparse_sketch_amd import configs as C
from long_context_sparse_sketch_amd.runtime import SparseDecodeLayer, StepRunner
from long_context_sparse_sketch_amd.synth import make_case
from tests.gpu_util import GpuCase, assert_attn_close, flush, lse_close, ref_arrays

pytestmark = pytest.mark.gpu

OUTS = ("S", "qsk", "qscale", "scores", "idx", "n_sel", "out", "lse")


# A byte pattern that wrecks any result it enters: bf16 / fp16 0x7B7B (about
# 1.3e36 / 6.1e4), int8 codes 0x7B = 123, int4 codes 7 and -5.
POISON = 0x7B


def build_tier(g: GpuCase, W_hot: int):
    """Pinned host copies of the cache and a device ring of the last W_hot
    positions of every sequence; returns (cache, host tensors, ring tensors)."""
    R = g.cfg.R
    host = [None if t is None else t.cpu().pin_memory() for t in (g.K, g.V, g.Ks, g.Vs)]
    ring = []
    for t in (g.K, g.V, g.Ks, g.Vs):
        if t is None:
            ring.append(None)
            continue
        r = torch.empty((t.shape[0], t.shape[1], W_hot) + tuple(t.shape[3:]), dtype=t.dtype,
                        device="cuda")
        r.view(torch.uint8).fill_(POISON)             # slots with no valid position
        for b in range(t.shape[0]):
            end = int(g.seq_len_np[b]) + R - 1                  # one past the last row's token
            pos = torch.arange(max(0, end - W_hot), end, device="cuda")
            r[b][:, pos % W_hot] = t[b][:, pos]
        ring.append(r)
    cache = sks.Cache(host[0], host[1], g.seq_len, host[2], host[3], hot=tuple(ring))
    return cache, host, ring


def poison_host(g: GpuCase, host):
    """Positions >= L_0 + R - 1 - window are inside every row's window (or past
    it): no row reads them from host."""
    R, W = g.cfg.R, g.window
    for t in host:
        if t is None:
            continue
        for b in range(t.shape[0]):
            start = max(0, int(g.seq_len_np[b]) + R - 1 - W)
            t[b][:, start:].view(torch.uint8).fill_(POISON)


def run(layer, q):
    for n in OUTS[1:]:
        getattr(layer, n).view(torch.uint8).fill_(0x5A)
    layer.step(q)
    torch.cuda.synchronize()
    return {n: getattr(layer, n).clone() for n in OUTS}


CASES = [
    (C.small(C.C3), None),
    (C.with_kv(C.small(C.C3), C.KV_I4), None),
    (C.small(C.C5), None),
    (C.with_kv(C.small(C.C5), C.KV_I4), None),
    (C.small(C.C2), 0.6),      # short rows: part of the ring holds no valid position
]


@pytest.mark.parametrize("cfg,short", CASES, ids=[c.name + ("_short" if s else "") for c, s in CASES])
def test_host_tier_equals_device_cache(cfg, short):
    case = make_case(cfg)
    B = case.B
    sl = np.array([cfg.L - 997 * b for b in range(B)], np.int32)      # ragged
    if short:
        sl = np.array([int(cfg.window * short) + 13 * b for b in range(B)], np.int32)
    flush(f"[tier] {cfg.name}: lengths {sl.tolist()}")
    g = GpuCase(case, seq_len=sl)
    g.layer.build_sketch(0, g.T)
    want = run(g.layer, g.q)

    W_hot = g.window + cfg.R + 37                                      # slots wrap unaligned
    cache, host, ring = build_tier(g, W_hot)
    lay = SparseDecodeLayer(B, cfg.R, cfg.Hq, cfg.Hkv, g.T, g.window, g.topk, g.pool,
                            cfg.kv_dtype).bind(cache, g.basis, g.key_scale)
    lay.build_sketch(0, g.T)                          # bulk build from host memory (clean)
    torch.cuda.synchronize()
    # the bulk build read the same bytes: the same codes as a device build
    # (g's own sketch has been through the step's APPEND since)
    g2 = GpuCase(case, seq_len=sl)
    g2.layer.build_sketch(0, g.T)
    torch.cuda.synchronize()
    assert torch.equal(lay.S, g2.layer.S), "bulk sketch from host memory"

    poison_host(g, host)
    got = run(lay, g.q)
    for n in OUTS:
        assert torch.equal(want[n].view(torch.uint8), got[n].view(torch.uint8)), n

    # and against the oracle on a few heads
    heads = [(b, h) for b in range(B) for h in range(min(cfg.Hkv, 2))]
    ref = g.oracle(heads=heads)
    arr = ref_arrays(ref, cfg, B, g.topk, g.layer.NB)
    out, lse = got["out"].cpu().numpy(), got["lse"].cpu().numpy()
    for (b, h) in heads:
        sl_h = slice(h * cfg.g, (h + 1) * cfg.g)
        assert_attn_close(out[b, :, sl_h], arr["out"][b, :, sl_h], f"{cfg.name} {(b, h)}")
        lse_close(lse[b, :, sl_h], arr["lse"][b, :, sl_h], f"{cfg.name} {(b, h)}")


def test_host_tier_gather_pack_and_graph_replay():
    cfg = C.with_kv(C.small(C.C5), C.KV_I4)
    case = make_case(cfg)
    g = GpuCase(case)
    g.layer.build_sketch(0, g.T)
    want = run(g.layer, g.q)
    cache, host, ring = build_tier(g, g.window + cfg.R + 5)
    lay = SparseDecodeLayer(case.B, cfg.R, cfg.Hq, cfg.Hkv, g.T, g.window, g.topk, g.pool,
                            cfg.kv_dtype).bind(cache, g.basis, g.key_scale)
    lay.S.copy_(g.layer.S)
    poison_host(g, host)
    # graph replays of the tiered step
    runner = StepRunner(lay)
    runner.capture(g.q)
    for rep in range(3):
        lay.out.zero_()
        lay.idx.fill_(-5)
        torch.cuda.synchronize()
        runner.replay()
        torch.cuda.synchronize()
        assert torch.equal(lay.out, want["out"]) and torch.equal(lay.idx, want["idx"]), rep
    # gather/pack: the same packed rows as from the device cache
    Cn = g.topk + g.window + g.pool - 1
    B, R, Hkv = case.B, cfg.R, cfg.Hkv
    row = case.K.shape[-1]
    outs = []
    for c in (g.cache, cache):
        Ko = torch.zeros((B, R, Hkv, Cn, row), dtype=torch.uint8, device="cuda")
        Vo = torch.zeros_like(Ko)
        Kso = torch.zeros((B, R, Hkv, Cn), dtype=torch.int16, device="cuda")
        Vso = torch.zeros_like(Kso)
        n_out = torch.zeros((B, R, Hkv), dtype=torch.int32, device="cuda")
        sks.gather_pack(c, lay.p, want["idx"], Ko, Vo, n_out, None, None, Kso, Vso)
        torch.cuda.synchronize()
        outs.append((Ko, Vo, Kso, Vso, n_out))
    for a, b in zip(*outs):
        assert torch.equal(a, b)


def test_host_tier_full_size_int4():
    """The benchmark's shape (8 x 250K, int4, graph-replayed step as bench.py
    --kv int4 --host-kv times it): bit-equal to the all-device step."""
    cfg = C.with_kv(C.C3, C.KV_I4)
    flush(f"[tier] full size {cfg.name}")
    case = make_case(cfg)
    g = GpuCase(case)
    g.layer.build_sketch(0, g.T)
    # the same poison in both runs' outputs: entries the step leaves undefined
    # (scores past the far region) then compare equal too
    for n in OUTS[1:]:
        getattr(g.layer, n).view(torch.uint8).fill_(0x5A)
    runner = StepRunner(g.layer)
    runner.capture(g.q)
    runner.replay()
    torch.cuda.synchronize()
    want = {n: getattr(g.layer, n).clone() for n in OUTS}
    cache, host, ring = build_tier(g, g.window + cfg.R)
    lay = SparseDecodeLayer(case.B, cfg.R, cfg.Hq, cfg.Hkv, g.T, g.window, g.topk, g.pool,
                            cfg.kv_dtype).bind(cache, g.basis, g.key_scale)
    lay.S.copy_(g.layer.S)
    poison_host(g, host)
    for n in OUTS[1:]:
        getattr(lay, n).view(torch.uint8).fill_(0x5A)
    runner = StepRunner(lay)
    runner.capture(g.q)
    runner.replay()
    torch.cuda.synchronize()
    for n in OUTS:
        assert torch.equal(want[n].view(torch.uint8), getattr(lay, n).view(torch.uint8)), n


@pytest.mark.parametrize("short", [True, False], ids=["within_window_plus_topk", "long"])
def test_host_tier_dense_step(short):
    """A dense step attends the last window + topk tokens, more than the ring
    holds: the positions older than the ring come from host memory, the rest
    from the ring (the host copy of the latter is poisoned)."""
    cfg = C.small(C.C3)
    case = make_case(cfg)
    B = case.B
    if short:     # longer than the ring, within window + topk
        sl = np.array([cfg.window + cfg.topk - 3 - 211 * b for b in range(B)], np.int32)
    else:
        sl = np.array([cfg.L - 5 * b for b in range(B)], np.int32)
    g = GpuCase(case, seq_len=sl)
    g.layer.build_sketch(0, g.T)
    for n in OUTS[1:]:
        getattr(g.layer, n).view(torch.uint8).fill_(0x5A)
    g.layer.step(g.q, dense=True)
    torch.cuda.synchronize()
    want = {n: getattr(g.layer, n).clone() for n in OUTS}
    W_hot = g.window + cfg.R + 37
    assert int(sl.min()) > W_hot
    cache, host, ring = build_tier(g, W_hot)
    lay = SparseDecodeLayer(B, cfg.R, cfg.Hq, cfg.Hkv, g.T, g.window, g.topk, g.pool,
                            cfg.kv_dtype).bind(cache, g.basis, g.key_scale)
    lay.S.copy_(g.layer.S)
    poison_host(g, host)
    for n in OUTS[1:]:
        getattr(lay, n).view(torch.uint8).fill_(0x5A)
    lay.step(g.q, dense=True)
    torch.cuda.synchronize()
    for n in OUTS:
        assert torch.equal(want[n].view(torch.uint8), getattr(lay, n).view(torch.uint8)), n


@pytest.mark.parametrize("seed", range(30))
def test_random_shape_host_tier(seed):
    """Seeded random shapes (unpooled: a hot tier needs pool == 1) with a ring
    of window + rows + 0..63 slots: every output bit-equal to the all-device
    run, the host copy of every position the rows may not read from host
    poisoned."""
    from tests.test_gpu_random_shapes import draw
    cfg, sl = draw(seed)
    if cfg.pool > 1:
        cfg = cfg.scaled(pool=1)
    if cfg.window + cfg.R > cfg.T_max:        # the ring may not exceed the cache
        cfg = cfg.scaled(window=cfg.T_max - cfg.R)
    extra = int(np.random.default_rng(900 + seed).integers(0, 64))
    flush(f"[tier random] seed {seed}: B={cfg.B} R={cfg.R} Hq/Hkv={cfg.Hq}/{cfg.Hkv} "
          f"L={sl.tolist()} W={cfg.window} k={cfg.topk} kv={C.KV_NAMES[cfg.kv_dtype]} "
          f"ring +{extra}")
    case = make_case(cfg)
    g = GpuCase(case, seq_len=sl)
    g.layer.build_sketch(0, g.T)
    S0 = g.layer.S.clone()
    want = run(g.layer, g.q)
    W_hot = min(g.window + cfg.R + extra, g.T)
    cache, host, ring = build_tier(g, W_hot)
    lay = SparseDecodeLayer(case.B, cfg.R, cfg.Hq, cfg.Hkv, g.T, g.window, g.topk, 1,
                            cfg.kv_dtype).bind(cache, g.basis, g.key_scale)
    lay.S.copy_(S0)
    poison_host(g, host)
    got = run(lay, g.q)
    for n in OUTS:
        assert torch.equal(want[n].view(torch.uint8), got[n].view(torch.uint8)), n
