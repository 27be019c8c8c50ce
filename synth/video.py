"""Seeded generator of video-shaped Q/K/V tensors.

Recipe (the same for every configuration):

* An embedding E[n, c] over the latent token grid: channel c follows one grid
  axis a = c mod 3 (t, h or w) with extent L_a; its wavelength is
  lambda_c = exp(U(ln 4, ln 4 L_a)) and its phase phi_c = U(0, 2 pi);
  E[n, c] = sin(2 pi pos_a(n) / lambda_c + phi_c).  E is shared by Q, K, V and
  by every batch and head, so neighbouring tokens (and blocks) correlate.
* X[b, h, n, c] = sigma * Z + a_h * E[n, c] for X in {Q, K, V}, with Z i.i.d.
  N(0, 1) drawn per (tensor, b, h).
* Optionally a set of "hot" block positions (shared by all b, h) gets +offset on
  every channel of Q, K and V, which creates long-range hot blocks.
* bf16 configurations round fp32 -> bf16 once with round-to-nearest-even;
  fp32 configurations keep the fp32 values.

Tokens are flattened in raster order n = (t * Hh + h) * W + w, and blocks tile
the grid from the origin with stride (bt, bh, bw); the last block along an
axis that the block size does not divide is partial.  The hot-block choice
needs that block numbering, which is restated here as plain index arithmetic
(no summaries, scores or attention).

Random streams: numpy PCG64 seeded with [seed, stream, ...]:
  3 = embedding, 4 = head amplitudes, 5 = hot blocks, 10 + x = Z for
  x = 0/1/2 (Q/K/V), indexed further by (b, h).
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace
from typing import List, Optional, Sequence

import numpy as np

MODE_COUNT = "count"
MODE_RATIO = "ratio"
MODE_MASS = "mass"


@dataclass(frozen=True)
class Config:
    name: str
    B: int
    H: int
    d: int
    T: int
    Hh: int
    W: int
    bt: int
    bh: int
    bw: int
    dtype: str  # "bf16" or "f32"
    sigma: float
    amp_kind: str  # "const", "uniform", "split"
    amp_params: tuple
    mode: str  # count / ratio / mass
    budget: tuple  # one value per head (len H) or a single value
    seed: int
    hot_frac: float = 0.0
    hot_offset: float = 0.0

    @property
    def N(self) -> int:
        return self.T * self.Hh * self.W

    @property
    def grid_blocks(self):
        return (
            -(-self.T // self.bt),
            -(-self.Hh // self.bh),
            -(-self.W // self.bw),
        )

    @property
    def nblk(self) -> int:
        a, b, c = self.grid_blocks
        return a * b * c

    def per_head_budget(self) -> List[float]:
        if len(self.budget) == 1:
            return [float(self.budget[0])] * self.H
        assert len(self.budget) == self.H
        return [float(x) for x in self.budget]

    def with_budget(self, mode: str, value) -> "Config":
        vals = tuple(value) if isinstance(value, (list, tuple)) else (float(value),)
        return replace(self, mode=mode, budget=vals, name=f"{self.name}[{mode}={value}]")

    def with_heads(self, H: int) -> "Config":
        return replace(self, H=H, name=f"{self.name}[H={H}]")


# The five workloads: tiny case, small/mid/large video layers, ragged stress.
CONFIGS = {
    "tiny": Config("tiny", B=1, H=2, d=64, T=4, Hh=8, W=8, bt=2, bh=4, bw=4,
                   dtype="f32", sigma=0.5, amp_kind="const", amp_params=(1.0,),
                   mode=MODE_COUNT, budget=(3,), seed=101),
    "small": Config("small", B=1, H=12, d=128, T=21, Hh=30, W=52, bt=3, bh=6, bw=4,
                    dtype="bf16", sigma=0.5, amp_kind="uniform", amp_params=(0.3, 2.0),
                    mode=MODE_RATIO, budget=(0.25,), seed=202),
    "mid": Config("mid", B=1, H=40, d=128, T=21, Hh=45, W=80, bt=3, bh=5, bw=8,
                  dtype="bf16", sigma=0.5, amp_kind="uniform", amp_params=(0.3, 2.0),
                  mode=MODE_MASS, budget=(0.9,), seed=303, hot_frac=0.02, hot_offset=3.0),
    "large": Config("large", B=1, H=24, d=128, T=33, Hh=45, W=80, bt=3, bh=5, bw=8,
                    dtype="bf16", sigma=0.5, amp_kind="split", amp_params=(12, 2.0, 0.3),
                    mode=MODE_RATIO, budget=(0.15,), seed=404),
    "ragged": Config("ragged", B=2, H=16, d=128, T=13, Hh=27, W=48, bt=4, bh=4, bw=4,
                     dtype="bf16", sigma=1.0, amp_kind="const", amp_params=(0.0,),
                     mode=MODE_RATIO, budget=(1.0,), seed=505),
}

# Reduced shapes that the fp64 oracle finishes in seconds; they still span
# several tiles, partial blocks along every axis and the degenerate cases.
TEST_CONFIGS = {
    "tiny": CONFIGS["tiny"],
    "tiny_bf16": replace(CONFIGS["tiny"], name="tiny_bf16", dtype="bf16"),
    # 48-token blocks, partial along t, h and w (7/3, 10/4, 13/4).
    "ragged_p64": Config("ragged_p64", B=1, H=3, d=128, T=7, Hh=10, W=13, bt=3, bh=4, bw=4,
                         dtype="bf16", sigma=0.5, amp_kind="uniform", amp_params=(0.3, 2.0),
                         mode=MODE_RATIO, budget=(0.3,), seed=11),
    # the mid block shape (120 tokens) with a partial last block along w and hot blocks.
    "mid_shape": Config("mid_shape", B=1, H=2, d=128, T=6, Hh=10, W=20, bt=3, bh=5, bw=8,
                        dtype="bf16", sigma=0.5, amp_kind="uniform", amp_params=(0.3, 2.0),
                        mode=MODE_MASS, budget=(0.9,), seed=12, hot_frac=0.1, hot_offset=3.0),
    # the small block shape (72 tokens).
    "small_shape": Config("small_shape", B=1, H=2, d=128, T=6, Hh=12, W=12, bt=3, bh=6, bw=4,
                          dtype="bf16", sigma=0.5, amp_kind="uniform", amp_params=(0.3, 2.0),
                          mode=MODE_RATIO, budget=(0.25,), seed=13),
    # ragged-stress block (4x4x4) with partial blocks, two batches.
    "ragged_small": Config("ragged_small", B=2, H=2, d=128, T=5, Hh=7, W=9, bt=4, bh=4, bw=4,
                           dtype="bf16", sigma=1.0, amp_kind="const", amp_params=(0.0,),
                           mode=MODE_RATIO, budget=(0.5,), seed=14),
    # blocks larger than one 128-query tile (256 tokens).
    "big_block": Config("big_block", B=1, H=2, d=128, T=8, Hh=16, W=16, bt=4, bh=8, bw=8,
                        dtype="bf16", sigma=0.5, amp_kind="const", amp_params=(1.0,),
                        mode=MODE_COUNT, budget=(3,), seed=15),
    # one token per block: token-level selection.
    "token_level": Config("token_level", B=1, H=2, d=128, T=4, Hh=4, W=8, bt=1, bh=1, bw=1,
                          dtype="bf16", sigma=0.5, amp_kind="const", amp_params=(1.0,),
                          mode=MODE_COUNT, budget=(5,), seed=16),
    # a single block covering the grid: dense attention.
    "one_block": Config("one_block", B=1, H=2, d=128, T=2, Hh=4, W=8, bt=2, bh=4, bw=8,
                        dtype="bf16", sigma=0.5, amp_kind="const", amp_params=(1.0,),
                        mode=MODE_COUNT, budget=(1,), seed=17),
    # head dimension 64 in bf16.
    "d64": Config("d64", B=1, H=2, d=64, T=6, Hh=10, W=16, bt=3, bh=5, bw=8,
                  dtype="bf16", sigma=0.5, amp_kind="uniform", amp_params=(0.3, 2.0),
                  mode=MODE_MASS, budget=(0.8,), seed=18),
    # the supported limits: 4096 blocks per head (one token each), a block
    # count between 2048 and 4096, and 1024-token blocks.
    "max_blocks": Config("max_blocks", B=1, H=1, d=64, T=16, Hh=16, W=16, bt=1, bh=1, bw=1,
                         dtype="bf16", sigma=0.5, amp_kind="const", amp_params=(1.0,),
                         mode=MODE_COUNT, budget=(8,), seed=20),
    "blocks_2k": Config("blocks_2k", B=1, H=1, d=128, T=12, Hh=12, W=12, bt=1, bh=1, bw=1,
                        dtype="bf16", sigma=0.5, amp_kind="const", amp_params=(1.0,),
                        mode=MODE_MASS, budget=(0.3,), seed=21),
    "max_block_tokens": Config("max_block_tokens", B=1, H=1, d=128, T=8, Hh=32, W=32, bt=4, bh=16, bw=16,
                               dtype="bf16", sigma=0.5, amp_kind="const", amp_params=(1.0,),
                               mode=MODE_COUNT, budget=(3,), seed=22),
    # 56-token blocks (a full 32-key subtile, then 24 keys) with 24-token
    # partial blocks along w (17 = 7 + 7 + 3).
    "tail24": Config("tail24", B=1, H=2, d=128, T=4, Hh=8, W=17, bt=2, bh=4, bw=7,
                     dtype="bf16", sigma=0.5, amp_kind="uniform", amp_params=(0.3, 2.0),
                     mode=MODE_MASS, budget=(0.7,), seed=23),
    # 120-token blocks and no partial block (3 x 3 x 3 blocks), hot blocks.
    "mid_full": Config("mid_full", B=1, H=2, d=128, T=9, Hh=15, W=24, bt=3, bh=5, bw=8,
                       dtype="bf16", sigma=0.5, amp_kind="uniform", amp_params=(0.3, 2.0),
                       mode=MODE_MASS, budget=(0.9,), seed=24, hot_frac=0.1, hot_offset=3.0),
    # Blocks whose tokens are a multiple of 8 (at least 32) everywhere but
    # would waste 16 or more keys padded to 32-key subtiles, so attention
    # streams the kept blocks' keys back to back: 72- and 40-token blocks
    # (partial along w; subtiles straddle block boundaries) ...
    "dense_mixed": Config("dense_mixed", B=1, H=3, d=128, T=6, Hh=12, W=23, bt=2, bh=4, bw=9,
                          dtype="bf16", sigma=0.5, amp_kind="uniform", amp_params=(0.3, 2.0),
                          mode=MODE_RATIO, budget=(0.4,), seed=25),
    # ... and 40-token blocks at head dimension 64, two batches.
    "dense_40": Config("dense_40", B=2, H=2, d=64, T=4, Hh=10, W=24, bt=1, bh=5, bw=8,
                       dtype="bf16", sigma=0.5, amp_kind="uniform", amp_params=(0.3, 2.0),
                       mode=MODE_MASS, budget=(0.8,), seed=26),
    # row counts on both sides of the one-kernel CSR build's limit (32768
    # rows): 512 and 513 heads of 64 one-token blocks.
    "rows_32k": Config("rows_32k", B=2, H=256, d=64, T=4, Hh=4, W=4, bt=1, bh=1, bw=1,
                       dtype="bf16", sigma=0.5, amp_kind="uniform", amp_params=(0.3, 2.0),
                       mode=MODE_MASS, budget=(0.6,), seed=27),
    "rows_32k_plus": Config("rows_32k_plus", B=3, H=171, d=64, T=4, Hh=4, W=4, bt=1, bh=1, bw=1,
                            dtype="bf16", sigma=0.5, amp_kind="uniform", amp_params=(0.3, 2.0),
                            mode=MODE_RATIO, budget=(0.3,), seed=28),
    # fp32 (debug) path on a ragged shape.
    "ragged_f32": Config("ragged_f32", B=1, H=2, d=128, T=5, Hh=7, W=9, bt=4, bh=4, bw=4,
                         dtype="f32", sigma=1.0, amp_kind="const", amp_params=(0.0,),
                         mode=MODE_RATIO, budget=(0.5,), seed=19),
}


def get_config(name: str) -> Config:
    if name in CONFIGS:
        return CONFIGS[name]
    return TEST_CONFIGS[name]


# ---------------------------------------------------------------------------
# bf16 bit helpers (storage conversion only)
# ---------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 -> bf16 with round-to-nearest-even; returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f32(b).astype(np.float64)


# ---------------------------------------------------------------------------
# generator
# ---------------------------------------------------------------------------

def _rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(list(key)))


def _embedding(cfg: Config) -> np.ndarray:
    """E[n, c] (fp32, [N, d]) from stream 3."""
    rng = _rng(cfg.seed, 3)
    ext = (cfg.T, cfg.Hh, cfg.W)
    u = rng.uniform(size=(cfg.d, 2))
    t = np.arange(cfg.T, dtype=np.float64)[:, None, None]
    h = np.arange(cfg.Hh, dtype=np.float64)[None, :, None]
    w = np.arange(cfg.W, dtype=np.float64)[None, None, :]
    pos = (t, h, w)
    E = np.empty((cfg.T, cfg.Hh, cfg.W, cfg.d), dtype=np.float32)
    for c in range(cfg.d):
        a = c % 3
        L = ext[a]
        lam = math.exp(math.log(4.0) + u[c, 0] * (math.log(4.0 * L) - math.log(4.0)))
        phi = 2.0 * math.pi * u[c, 1]
        val = np.sin(2.0 * math.pi * pos[a] / lam + phi)
        E[..., c] = np.broadcast_to(val, (cfg.T, cfg.Hh, cfg.W))
    return E.reshape(cfg.N, cfg.d)


def head_amplitudes(cfg: Config) -> np.ndarray:
    if cfg.amp_kind == "const":
        return np.full(cfg.H, float(cfg.amp_params[0]))
    if cfg.amp_kind == "uniform":
        lo, hi = cfg.amp_params
        return _rng(cfg.seed, 4).uniform(lo, hi, size=cfg.H)
    if cfg.amp_kind == "split":
        h0, a0, a1 = cfg.amp_params
        return np.array([a0 if h < h0 else a1 for h in range(cfg.H)], dtype=np.float64)
    raise ValueError(cfg.amp_kind)


def hot_token_mask(cfg: Config) -> Optional[np.ndarray]:
    """Boolean [N] mask of tokens inside the hot block positions (stream 5)."""
    if cfg.hot_frac <= 0.0:
        return None
    nT, nH, nW = cfg.grid_blocks
    nblk = nT * nH * nW
    n_hot = max(1, int(round(cfg.hot_frac * nblk)))
    hot = _rng(cfg.seed, 5).choice(nblk, size=n_hot, replace=False)
    mask = np.zeros((cfg.T, cfg.Hh, cfg.W), dtype=bool)
    for j in hot.tolist():
        it, rem = divmod(j, nH * nW)
        ih, iw = divmod(rem, nW)
        mask[it * cfg.bt:(it + 1) * cfg.bt,
             ih * cfg.bh:(ih + 1) * cfg.bh,
             iw * cfg.bw:(iw + 1) * cfg.bw] = True
    return mask.reshape(cfg.N)


def make_inputs(cfg: Config, threads: int = 8, heads: Optional[Sequence[int]] = None):
    """Return dict with 'q', 'k', 'v' as numpy arrays [B, H', N, d].

    bf16 configs give uint16 bit patterns, f32 configs give float32.  `heads`
    restricts generation to a subset of heads (same values as the full run).
    """
    E = _embedding(cfg)
    amps = head_amplitudes(cfg)
    hot = hot_token_mask(cfg)
    head_list = list(range(cfg.H)) if heads is None else list(heads)
    out_dtype = np.uint16 if cfg.dtype == "bf16" else np.float32
    out = {
        name: np.empty((cfg.B, len(head_list), cfg.N, cfg.d), dtype=out_dtype)
        for name in ("q", "k", "v")
    }

    def one(job):
        x, name, b, hi = job
        h = head_list[hi]
        z = _rng(cfg.seed, 10 + x, b, h).standard_normal(size=(cfg.N, cfg.d), dtype=np.float32)
        val = np.float32(cfg.sigma) * z + np.float32(amps[h]) * E
        if hot is not None:
            val[hot] += np.float32(cfg.hot_offset)
        if cfg.dtype == "bf16":
            out[name][b, hi] = f32_to_bf16_bits(val)
        else:
            out[name][b, hi] = val

    jobs = [(x, name, b, hi) for x, name in enumerate(("q", "k", "v"))
            for b in range(cfg.B) for hi in range(len(head_list))]
    if threads > 1 and len(jobs) > 1:
        with ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(one, jobs))
    else:
        for j in jobs:
            one(j)
    return out
