"""Seeded synthetic inputs for MLA decode (weights, new hidden states, cached rows).

This module is shared by the GPU path's tests and benchmark and by the CPU
oracle's tests. It holds none of the method's arithmetic: it only draws random
numbers, rounds them to the storage dtype and lays them out in memory. Cached
history rows are drawn directly from the distribution that compressing a
N(0, 1) hidden state through N(0, w_std^2) weights induces (each latent entry
and each rotary-key entry is N(0, w_std^2 * d); a rotation leaves an isotropic
Gaussian unchanged, so no position dependent arithmetic is needed here).

Geometry follows the DeepSeek-V3 numbers the pages use ("Understanding MLA",
section 3: hidden 7168, 128 heads, latent 512, rotary key 64, per-head
nope 128 and value 128; "Multi-Head Latent Attention" (llm-arch-kb), section 4:
query latent 1536, 61 layers).

Storage conventions:
  * bf16 arrays are numpy uint16 bit patterns (round-to-nearest-even from the
    float32 draw); fp32 arrays are numpy float32.
  * Unused cache rows and unused page slots hold NaN, so a kernel that reads
    past a sequence's length produces NaN in its output.
"""
from __future__ import annotations

import dataclasses
import math
from dataclasses import dataclass, field
from typing import Optional, Sequence

import numpy as np

BF16_NAN = np.uint16(0x7FC0)

# Order in which child random streams are spawned from the seed. Fixed so that
# every consumer draws identical values.
_STREAMS = ("W_DKV", "W_KR", "W_DQ", "W_UQ", "W_QR", "W_UK", "W_UV", "W_O",
            "h_t", "history", "ctx", "pages", "gamma", "q", "topk", "prefill_q")


@dataclass(frozen=True)
class MLAConfig:
    name: str
    d: int            # hidden width
    H: int            # query heads
    d_c: int          # KV latent width
    d_R: int          # decoupled rotary key width
    d_h: int          # per-head nope (content) query/key width
    d_v: int          # per-head value width
    d_cq: int         # query latent width; 0 = no query low-rank
    dtype: str        # storage dtype: "fp32" or "bf16"
    B: int            # sequences in the batch
    ctx: Optional[Sequence[int]] = None   # rows already cached, per sequence
    ctx_range: Optional[tuple] = None     # (lo, hi) inclusive, drawn per sequence
    paged: bool = False
    block_size: int = 64
    cap_pad: int = 0                      # extra NaN rows past the longest sequence
    theta: float = 10000.0
    w_std: float = 0.02
    softmax_scale: float = 0.0            # 0 -> 1/sqrt(d_h + d_R)
    gamma: bool = False                   # draw an RMSNorm weight for the latent
    topk: int = 0                         # > 0: attention over a listed top-k subset of rows
    seed: int = 0

    @property
    def D(self) -> int:
        return self.d_c + self.d_R

    @property
    def scale(self) -> float:
        if self.softmax_scale:
            return self.softmax_scale
        return 1.0 / math.sqrt(self.d_h + self.d_R)

    def with_(self, **kw) -> "MLAConfig":
        return dataclasses.replace(self, **kw)


_V3 = dict(d=7168, H=128, d_c=512, d_R=64, d_h=128, d_v=128, d_cq=1536,
           dtype="bf16")

# The five workloads the build is measured and checked on.
CONFIGS = {
    "tiny_fp32": MLAConfig(name="tiny_fp32", d=256, H=4, d_c=32, d_R=8, d_h=16,
                           d_v=16, d_cq=0, dtype="fp32", B=1, ctx=(64,),
                           softmax_scale=1.0 / math.sqrt(24)),
    "v3_b1_ctx4k": MLAConfig(name="v3_b1_ctx4k", B=1, ctx=(4096,), **_V3),
    "v3_b64_ctx8k": MLAConfig(name="v3_b64_ctx8k", B=64, ctx=(8192,) * 64, **_V3),
    "v3_b8_ctx32k": MLAConfig(name="v3_b8_ctx32k", B=8, ctx=(32768,) * 8, **_V3),
    "v3_b128_ragged_paged": MLAConfig(name="v3_b128_ragged_paged", B=128,
                                      ctx_range=(1024, 16384), paged=True,
                                      block_size=64, **_V3),
    # the RMS-normalised latent variant at the headline size
    "v3_b64_ctx8k_norm": MLAConfig(name="v3_b64_ctx8k_norm", B=64, ctx=(8192,) * 64, gamma=True, **_V3),
    # sparse attention over a top-2048 list per sequence at the headline size
    "v3_b64_ctx8k_topk2048": MLAConfig(name="v3_b64_ctx8k_topk2048", B=64, ctx=(8192,) * 64, topk=2048, **_V3),
    # causal prefill: the newest T tokens of 4 sequences of 4096 cached rows
    "v3_b4_ctx4k_prefill": MLAConfig(name="v3_b4_ctx4k_prefill", B=4, ctx=(4096,) * 4, **_V3),
}
CONFIG_ORDER = list(CONFIGS)


def _rngs(seed: int):
    kids = np.random.SeedSequence(seed).spawn(len(_STREAMS))
    return {n: np.random.default_rng(s) for n, s in zip(_STREAMS, kids)}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    """Decode uint16 bfloat16 bit patterns (exact) to float64."""
    b = np.asarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Stored values as float64 (exact for both storage dtypes)."""
    if dtype == "bf16":
        return bf16_bits_to_f64(a)
    return np.asarray(a, dtype=np.float32).astype(np.float64)


def _draw(rng, shape, std, dtype, chunk=1 << 24):
    """N(0, std^2) draw rounded once to the storage dtype."""
    n = int(np.prod(shape)) if len(shape) else 1
    out = np.empty(n, dtype=np.uint16 if dtype == "bf16" else np.float32)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        v = rng.standard_normal(e - s, dtype=np.float32)
        if std != 1.0:
            v *= np.float32(std)
        out[s:e] = f32_to_bf16_bits(v) if dtype == "bf16" else v
    return out.reshape(shape)


def _draw_cols(rng, shape, col_std, dtype):
    """N(0, col_std[j]^2) in column j of rows of shape [n][len(col_std)],
    rounded once to the storage dtype."""
    v = rng.standard_normal(shape, dtype=np.float32) * np.asarray(col_std, dtype=np.float32)
    return f32_to_bf16_bits(v) if dtype == "bf16" else v


def _nan_fill(shape, dtype):
    if dtype == "bf16":
        return np.full(shape, BF16_NAN, dtype=np.uint16)
    return np.full(shape, np.nan, dtype=np.float32)


def context_lengths(cfg: MLAConfig) -> np.ndarray:
    """Rows already cached per sequence (the new token goes at that position)."""
    if cfg.ctx is not None:
        ctx = np.asarray(cfg.ctx, dtype=np.int64)
        if ctx.size == 1 and cfg.B > 1:
            ctx = np.full(cfg.B, int(ctx[0]), dtype=np.int64)
        assert ctx.size == cfg.B
        return ctx
    lo, hi = cfg.ctx_range
    return _rngs(cfg.seed)["ctx"].integers(lo, hi + 1, size=cfg.B).astype(np.int64)


@dataclass
class MLAInputs:
    cfg: MLAConfig
    weights: dict                 # name -> stored array (None where absent)
    h_t: np.ndarray               # [B][d] new tokens' hidden states
    ctx: np.ndarray               # [B] rows already cached = new token's position
    seq_lens: np.ndarray          # [B] rows attended after the append = ctx + 1
    cache: np.ndarray             # contiguous [B][cap][D] or paged pool [n_blocks][bs][D]
    block_table: Optional[np.ndarray] = None   # [B][max_blocks] int32, -1 unused
    capacity: int = 0             # contiguous capacity (rows per sequence)
    extras: dict = field(default_factory=dict)

    def row(self, b: int, u: int) -> np.ndarray:
        """Stored cache row u of sequence b (a view)."""
        if self.block_table is None:
            return self.cache[b, u]
        bs = self.cfg.block_size
        return self.cache[self.block_table[b, u // bs], u % bs]

    def rows(self, b: int, n: int) -> np.ndarray:
        """First n stored rows of sequence b, [n][D] (a copy for paged caches)."""
        if self.block_table is None:
            return self.cache[b, :n]
        bs = self.cfg.block_size
        nb = (n + bs - 1) // bs
        pages = self.cache[self.block_table[b, :nb]].reshape(nb * bs, self.cache.shape[-1])
        return pages[:n]


def make_weights(cfg: MLAConfig) -> dict:
    r = _rngs(cfg.seed)
    s, dt = cfg.w_std, cfg.dtype
    q_in = cfg.d_cq if cfg.d_cq else cfg.d
    w = {
        "W_DKV": _draw(r["W_DKV"], (cfg.d_c, cfg.d), s, dt),
        "W_KR": _draw(r["W_KR"], (cfg.d_R, cfg.d), s, dt),
        "W_DQ": _draw(r["W_DQ"], (cfg.d_cq, cfg.d), s, dt) if cfg.d_cq else None,
        "W_UQ": _draw(r["W_UQ"], (cfg.H, cfg.d_h, q_in), s, dt),
        "W_QR": _draw(r["W_QR"], (cfg.H, cfg.d_R, q_in), s, dt),
        "W_UK": _draw(r["W_UK"], (cfg.H, cfg.d_h, cfg.d_c), s, dt),
        "W_UV": _draw(r["W_UV"], (cfg.H, cfg.d_v, cfg.d_c), s, dt),
        "W_O": _draw(r["W_O"], (cfg.d, cfg.H * cfg.d_v), s, dt),
        "gamma_kv": None,
    }
    if cfg.gamma:
        g = 1.0 + 0.1 * r["gamma"].standard_normal(cfg.d_c).astype(np.float32)
        w["gamma_kv"] = f32_to_bf16_bits(g) if dt == "bf16" else g
    return w


def make_inputs(cfg: MLAConfig, with_weights: bool = True) -> MLAInputs:
    """Seeded inputs for one decode step of cfg.

    The prior ctx[b] rows of every sequence are filled; the row at position
    ctx[b] (where the new token is appended) and everything past it is NaN.
    """
    r = _rngs(cfg.seed)
    dt, D = cfg.dtype, cfg.D
    ctx = context_lengths(cfg)
    seq_lens = ctx + 1
    hist_std = cfg.w_std * math.sqrt(cfg.d)
    weights = make_weights(cfg) if with_weights else {}
    h_t = _draw(r["h_t"], (cfg.B, cfg.d), 1.0, dt)
    hist = r["history"]
    if cfg.gamma:
        # latents stored by the normalised variant have unit RMS before the
        # gain: column j of the latent part ~ N(0, gamma_j^2); the rotary
        # part is not normalised
        g = to_f64(make_weights(cfg)["gamma_kv"], dt) if not with_weights else to_f64(weights["gamma_kv"], dt)
        col_std = np.concatenate([np.abs(g), np.full(cfg.d_R, hist_std)])

        def draw_hist(n):
            return _draw_cols(hist, (n, D), col_std, dt)
    else:
        def draw_hist(n):
            return _draw(hist, (n, D), hist_std, dt)
    if not cfg.paged:
        cap = int(seq_lens.max()) + cfg.cap_pad
        cache = _nan_fill((cfg.B, cap, D), dt)
        for b in range(cfg.B):
            n = int(ctx[b])
            if n:
                cache[b, :n] = draw_hist(n)
        return MLAInputs(cfg, weights, h_t, ctx, seq_lens, cache, None, cap)
    bs = cfg.block_size
    nblk = (seq_lens + bs - 1) // bs
    total = int(nblk.sum())
    perm = r["pages"].permutation(total).astype(np.int32)
    max_blocks = int(nblk.max())
    table = np.full((cfg.B, max_blocks), -1, dtype=np.int32)
    pool = _nan_fill((total, bs, D), dt)
    off = 0
    for b in range(cfg.B):
        nb = int(nblk[b])
        table[b, :nb] = perm[off:off + nb]
        off += nb
        n = int(ctx[b])
        if n:
            rows = draw_hist(n)
            full = n // bs
            if full:
                pool[table[b, :full]] = rows[:full * bs].reshape(full, bs, D)
            rem = n - full * bs
            if rem:
                pool[table[b, full], :rem] = rows[full * bs:]
    return MLAInputs(cfg, weights, h_t, ctx, seq_lens, pool, table, 0)


def make_topk_indices(cfg: MLAConfig, seq_lens: np.ndarray, topk: int):
    """A seeded top-k list per sequence, as a selector above the cache would
    hand it over: (indices [B][topk] int32, counts [B] int32). Sequence b
    lists min(topk, L_b) distinct positions of [0, L_b) in random order (the
    appended row among the candidates); unused entries are -1."""
    rng = _rngs(cfg.seed)["topk"]
    B = len(seq_lens)
    idx = np.full((B, topk), -1, dtype=np.int32)
    counts = np.minimum(np.asarray(seq_lens, dtype=np.int64), topk).astype(np.int32)
    for b in range(B):
        n = int(counts[b])
        idx[b, :n] = rng.choice(int(seq_lens[b]), size=n, replace=False).astype(np.int32)
    return idx, counts


def make_query(cfg: MLAConfig, q_std: float = 0.5) -> np.ndarray:
    """A seeded absorbed query [B][H][d_c + d_R] in the storage dtype, for
    exercising the attention call on its own (default std gives scores of
    about the spread a full V3-shaped step produces)."""
    return _draw(_rngs(cfg.seed)["q"], (cfg.B, cfg.H, cfg.D), q_std, cfg.dtype)


def make_prefill_query(cfg: MLAConfig, T: int, q_std: float = 1.0) -> np.ndarray:
    """A seeded per-head query [B][T][H][d_h + d_R] ([q_C ; q_R] per head) in the
    storage dtype for T prefill tokens per sequence (std 1 gives scores of a
    spread similar to the decode workloads against the history rows)."""
    return _draw(_rngs(cfg.seed)["prefill_q"], (cfg.B, T, cfg.H, cfg.d_h + cfg.d_R), q_std, cfg.dtype)
