"""The five workload shapes of the sparse-sketch decode-attention path.

Each record fixes the shape of one decode-attention step over one layer:
batch, query rows per sequence, query/KV heads, context length, exact window,
top-k, far-field pooling ratio and KV storage type.  Sources:

* "8 agents x 250K context, concurrently, on two 3090s" (r/LocalLLaMA post),
  claims list: each decode step reads ~1% of the tokens, picked with a rank-64
  key sketch; "What it took": pick the top ~2K.
* "Agens SGLang" README, "What it adds": a 4,096-token sliding window plus a
  4:1 mean-pooled far field merged under one softmax; "Quick start": the
  verify step of speculative decoding served as a chain.

`L` is the valid length seen by query row 0, including that row's own token
(its key/value is already in the cache).  Row i sees `L + i` tokens.
"""
from __future__ import annotations

from dataclasses import dataclass

HEAD_DIM = 128
RANK = 64

KV_BF16 = 0
KV_I8 = 1
KV_I4 = 2
KV_NAMES = {KV_BF16: "bf16", KV_I8: "int8", KV_I4: "int4"}


@dataclass(frozen=True)
class Config:
    name: str
    cid: int            # 1..5, also picks the seed (1000 + cid)
    B: int              # sequences
    R: int              # query rows per sequence (1 = plain decode)
    Hq: int
    Hkv: int
    L: int              # valid length of row 0 (includes its own token)
    window: int
    topk: int
    pool: int           # far-field pooling ratio r (1 = unpooled)
    kv_dtype: int       # KV_BF16, KV_I8 or KV_I4 (int8 / packed int4 + fp16 per-token scale)
    needle_kind: str    # how needles are planted (see synth.py)
    needle_count: int   # per sequence (clusters) or per KV head
    needle_amp: float
    needle_noise: float

    @property
    def D(self) -> int:
        return HEAD_DIM

    @property
    def rank(self) -> int:
        return RANK

    @property
    def g(self) -> int:
        return self.Hq // self.Hkv

    @property
    def kv_row_bytes(self) -> int:
        """Bytes of one cached K (or V) row, its scale excluded."""
        return {KV_BF16: 2 * HEAD_DIM, KV_I8: HEAD_DIM, KV_I4: HEAD_DIM // 2}[self.kv_dtype]

    @property
    def T_max(self) -> int:
        # room for every query row's own token
        return self.L + self.R - 1

    @property
    def seed(self) -> int:
        return 1000 + self.cid

    def row_len(self, i: int) -> int:
        return self.L + i

    def n_far(self, i: int) -> int:
        """Far tokens (r == 1) or far blocks (r > 1) of row i."""
        Li = self.row_len(i)
        return (Li - self.window) // self.pool if Li > self.window else 0

    def n_attended(self, i: int) -> int:
        """|U| for row i: selected far entries plus the exact window."""
        nf = self.n_far(i)
        k_eff = min(self.topk, nf)
        return k_eff + (self.row_len(i) - nf * self.pool)

    def scaled(self, **kw) -> "Config":
        d = dict(self.__dict__)
        d.update(kw)
        return Config(**d)


C1 = Config("tiny", 1, B=1, R=1, Hq=1, Hkv=1, L=4096, window=512, topk=256, pool=1,
            kv_dtype=KV_BF16, needle_kind="random", needle_count=16,
            needle_amp=3.0, needle_noise=0.5)
C2 = Config("qwen27b_like", 2, B=1, R=1, Hq=40, Hkv=8, L=32768, window=4096, topk=2048,
            pool=1, kv_dtype=KV_BF16, needle_kind="random", needle_count=64,
            needle_amp=2.5, needle_noise=0.5)
C3 = Config("multi_agent_250k", 3, B=8, R=1, Hq=24, Hkv=4, L=250000, window=4096,
            topk=2048, pool=1, kv_dtype=KV_BF16, needle_kind="clusters",
            needle_count=2500, needle_amp=2.5, needle_noise=0.5)
C4 = Config("bcsa_far_field", 4, B=16, R=1, Hq=32, Hkv=8, L=131072, window=4096,
            topk=1024, pool=4, kv_dtype=KV_BF16, needle_kind="blocks", needle_count=64,
            needle_amp=2.5, needle_noise=0.5)
C5 = Config("spec_verify_int8", 5, B=4, R=3, Hq=40, Hkv=8, L=65537, window=4096,
            topk=2048, pool=1, kv_dtype=KV_I8, needle_kind="row0", needle_count=64,
            needle_amp=2.5, needle_noise=0.5)

ALL = (C1, C2, C3, C4, C5)
BY_NAME = {c.name: c for c in ALL}


def small(cfg: Config) -> Config:
    """A reduced shape of `cfg` that the oracle finishes in seconds.

    Keeps the head layout, pooling, dtype and row count; shrinks batch,
    context, window and top-k so that every kernel still spans several
    tiles and a ragged tail.
    """
    if cfg.cid == 1:
        return cfg
    L = {2: 12345, 3: 20011, 4: 9000, 5: 7001}[cfg.cid]
    return cfg.scaled(name=cfg.name + "_small", B=min(cfg.B, 2), L=L,
                      window=min(cfg.window, 1000 + cfg.cid),
                      topk=min(cfg.topk, 700 if cfg.pool == 1 else 300),
                      needle_count=min(cfg.needle_count, 40 if cfg.cid != 3 else 150))


def full_set(cfg: Config) -> Config:
    """A reduced context with the workload's full attention set: the same
    window, top-k, pooling, rows, heads and dtype, a far region a little over
    twice top-k, and enough sequences for at least 512 attention workgroups
    of 384 entries (segments x splits): the workload's whole attention sets
    at a size the oracle finishes in seconds."""
    set_max = cfg.topk + cfg.window + cfg.pool - 1
    per_seq = cfg.R * cfg.Hkv * -(-set_max // 384)
    B = max(1, -(-512 // per_seq))
    L = cfg.window + 2 * cfg.topk * cfg.pool + 1234
    return cfg.scaled(name=cfg.name + "_full_set", B=B, L=L,
                      needle_count=min(cfg.needle_count, 40 if cfg.cid != 3 else 150))


def with_kv(cfg: Config, kv_dtype: int) -> Config:
    """`cfg` with another KV storage type (name suffixed with it unless it is
    the config's own).  The int4 cache is the one the claims list of "8
    agents x 250K context ..." keeps in host RAM; here it is a storage option
    of every shape.  Pooling needs a bf16 cache."""
    if kv_dtype == cfg.kv_dtype:
        return cfg
    if cfg.pool > 1 and kv_dtype != KV_BF16:
        raise ValueError(f"{cfg.name}: pooling needs a bf16 cache")
    base = cfg.name.replace("_" + KV_NAMES[cfg.kv_dtype], "")
    return cfg.scaled(name=f"{base}_{KV_NAMES[kv_dtype]}", kv_dtype=kv_dtype)
