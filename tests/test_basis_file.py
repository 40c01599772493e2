"""The frozen sketch basis file ("8 agents x 250K context ...", "What it took":
a frozen sketch basis in one file): byte layout, round trip and refusal of
malformed files.  CPU only."""
import struct

import numpy as np
import pytest

from long_context_sparse_sketch_amd import basis_file as bf


def _arrays(n, Hkv, seed=0):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((n, 64, 128)).astype(np.float32),
            rng.uniform(0.01, 1.0, Hkv).astype(np.float32))


@pytest.mark.parametrize("per_head,Hkv", [(True, 4), (False, 4), (False, 1), (True, 1)])
def test_round_trip_bit_exact(tmp_path, per_head, Hkv):
    b, ks = _arrays(Hkv if per_head else 1, Hkv)
    p = str(tmp_path / "basis.sksb")
    bf.save(p, b, ks, basis_per_head=per_head)
    b2, ks2, ph = bf.load(p)
    assert ph == per_head
    assert b2.dtype == np.float32 and ks2.dtype == np.float32
    assert np.array_equal(b2.view(np.uint32), b.view(np.uint32))
    assert np.array_equal(ks2.view(np.uint32), ks.view(np.uint32))


def test_byte_layout(tmp_path):
    """The documented layout, read back with plain struct unpacking."""
    b, ks = _arrays(2, 2, seed=3)
    p = str(tmp_path / "basis.sksb")
    bf.save(p, b, ks, basis_per_head=True)
    raw = open(p, "rb").read()
    assert raw[:8] == b"SKSBASIS"
    assert struct.unpack_from("<5i", raw, 8) == (1, 1, 2, 64, 128)
    assert raw[28:64] == b"\0" * 36
    assert len(raw) == 64 + 4 * (2 * 64 * 128 + 2)
    assert struct.unpack_from("<f", raw, 64)[0] == b[0, 0, 0]
    assert struct.unpack_from("<f", raw, 64 + 4 * (64 * 128 + 5))[0] == b[1, 0, 5]
    assert struct.unpack_from("<2f", raw, 64 + 4 * 2 * 64 * 128) == tuple(ks.tolist())


def test_shape_inference_and_2d_basis(tmp_path):
    b, ks = _arrays(1, 3)
    p = str(tmp_path / "b.sksb")
    bf.save(p, b[0], ks)                       # [rank][D]: one shared basis
    b2, _, ph = bf.load(p)
    assert not ph and b2.shape == (1, 64, 128)
    b4, ks4 = _arrays(3, 3)
    bf.save(p, b4, ks4)                        # one basis per head, inferred
    assert bf.load(p)[2]


def test_save_refuses_inconsistent_arrays(tmp_path):
    p = str(tmp_path / "b.sksb")
    b, ks = _arrays(3, 4)
    with pytest.raises(bf.BasisFileError):
        bf.save(p, b, ks, basis_per_head=True)             # 3 bases, 4 heads
    b1, ks1 = _arrays(1, 2)
    with pytest.raises(bf.BasisFileError):
        bf.save(p, b1, np.array([0.1, 0.0], np.float32))     # a zero key scale
    with pytest.raises(bf.BasisFileError):
        bf.save(p, b1, np.array([0.1, np.nan], np.float32))
    bad = b1.copy()
    bad[0, 3, 7] = np.inf
    with pytest.raises(bf.BasisFileError):
        bf.save(p, bad, ks1)


def test_load_refuses_malformed_files(tmp_path):
    b, ks = _arrays(2, 2)
    p = str(tmp_path / "b.sksb")
    bf.save(p, b, ks, basis_per_head=True)
    good = open(p, "rb").read()

    def check(raw):
        q = str(tmp_path / "bad.sksb")
        open(q, "wb").write(raw)
        with pytest.raises(bf.BasisFileError):
            bf.load(q)

    check(good[:40])                                        # truncated header
    check(b"NOTBASIS" + good[8:])                           # magic
    check(good[:8] + struct.pack("<i", 2) + good[12:])      # version
    check(good[:12] + struct.pack("<i", 5) + good[16:])     # basis_per_head not 0/1
    check(good[:40] + b"\1" + good[41:])                    # reserved byte
    check(good[:-4])                                        # truncated body
    check(good + b"\0\0\0\0")                               # trailing bytes
    neg = bytearray(good)
    struct.pack_into("<f", neg, len(good) - 4, -0.5)        # negative key scale
    check(bytes(neg))
