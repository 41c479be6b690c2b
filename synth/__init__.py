"""Seeded synthetic inputs for packed variable-length causal attention.

This module produces the two things every run needs and nothing else:

* sample lengths (and the ``cu_seqlens`` prefix array) for one packed
  sequence of ``L`` tokens, and
* bf16 tensors (held as ``uint16`` bit patterns) drawn from N(0, 1), and
  seeded variants of them whose logits leave the N(0, 1) range (scaled,
  rising or falling along each sample) for the numerics tests.

It holds none of the attention arithmetic.  Both the fp64 oracle (``oracle/``)
and the HIP path consume what it returns, so the two sides see identical bits.

Length recipe.  The pages' corpora are proprietary; their raw-sample lengths
are long-tailed with a median of 644 tokens and a p99 around 71K tokens
(Libra technical review, section 3.1; Libra paper, section 1).  The stand-in is
a lognormal with median 644 and sigma 2.0: lengths are drawn one at a time as
``clamp(round(exp(ln 644 + 2.0 z)), 1, L)`` and appended while the running sum
is below ``L``; the last draw is cut so the pack holds exactly ``L`` tokens.
Skewed packs place a fixed long sample first and fill the rest the same way.

Tensor recipe.  Each tensor (q, k, v, dout) is drawn in chunks of 2**20
elements; chunk ``c`` of tensor ``t`` uses its own PCG64 stream seeded by
``SeedSequence(entropy=seed, spawn_key=(t, c))``, draws fp32 N(0, 1) and rounds
it to bf16 with round-to-nearest-even.  The result does not depend on how many
threads generate the chunks.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

LOGNORMAL_MEDIAN = 644
LOGNORMAL_SIGMA = 2.0
CHUNK = 1 << 20

TENSOR_IDS = {"q": 1, "k": 2, "v": 3, "dout": 4}


@dataclass(frozen=True)
class Workload:
    """One packed-sequence attention workload (shape, tiling and length recipe)."""

    name: str
    total_tokens: int          # L
    h_q: int
    h_kv: int
    head_dim: int
    tile_tokens: int           # SH-Tile sequence block B
    tile_heads: int            # SH-Tile head-shard width (h_q / H)
    fixed_lengths: tuple = ()  # exact lengths (used alone when fill is False)
    first_lengths: tuple = ()  # long samples placed first, then lognormal filler
    fill: bool = True
    backward: bool = False

    def with_tokens(self, total_tokens: int, first_lengths: tuple = None, name: str = None):
        """Same shape and tiling at a different L (for small parity cases)."""
        return Workload(
            name=name or f"{self.name}@{total_tokens}",
            total_tokens=total_tokens, h_q=self.h_q, h_kv=self.h_kv,
            head_dim=self.head_dim, tile_tokens=self.tile_tokens,
            tile_heads=self.tile_heads, fixed_lengths=(),
            first_lengths=self.first_lengths if first_lengths is None else first_lengths,
            fill=True, backward=self.backward)


WORKLOADS = {
    w.name: w
    for w in [
        # 2K tokens, four samples, 4 Q / 4 KV heads, d = 64, SH-Tiles 256 x 2.
        Workload("tiny_2k", 2048, 4, 4, 64, 256, 2, fixed_lengths=(1024, 512, 256, 256), fill=False),
        # Qwen3-8B-shaped 32K pack: 32 Q / 8 KV heads, d = 128, SH-Tiles 4096 x 8.
        Workload("gqa_32k", 32768, 32, 8, 128, 4096, 8),
        # Skew pair at 128K, 30B-A3B shape (32 Q / 4 KV): one 40960-token sample + filler ...
        Workload("skew_128k_a", 131072, 32, 4, 128, 4096, 8, first_lengths=(40960,)),
        # ... versus 32 samples of 4096 tokens (equal L).
        Workload("skew_128k_b", 131072, 32, 4, 128, 4096, 8, fixed_lengths=(4096,) * 32, fill=False),
        # 1M-token pack, one GPU's head share of a 64 Q / 4 KV model: 8 Q / 1 KV heads.
        Workload("share_1m", 1048576, 8, 1, 128, 8192, 2, first_lengths=(600000,)),
        # 256K pack, 32 Q / 4 KV heads, forward and backward, SH-Tiles 8192 x 4.
        Workload("train_256k", 262144, 32, 4, 128, 8192, 4, backward=True),
    ]
}


def lognormal_fill(rng: np.random.Generator, remaining: int, cap: int) -> list:
    """Lognormal(median 644, sigma 2.0) lengths appended until ``remaining`` is used up."""
    out = []
    mu = math.log(LOGNORMAL_MEDIAN)
    while remaining > 0:
        z = rng.standard_normal()
        ell = int(round(math.exp(mu + LOGNORMAL_SIGMA * z)))
        ell = max(1, min(ell, cap))
        ell = min(ell, remaining)
        out.append(ell)
        remaining -= ell
    return out


def make_lengths(w: Workload, seed: int) -> np.ndarray:
    """Sample lengths (int64) of the pack; they sum to exactly ``w.total_tokens``."""
    L = w.total_tokens
    lengths = list(w.fixed_lengths) + list(w.first_lengths)
    used = sum(lengths)
    if used > L:
        raise ValueError(f"fixed lengths {used} exceed L={L}")
    if w.fill and used < L:
        rng = np.random.default_rng(seed)
        lengths += lognormal_fill(rng, L - used, L)
    if sum(lengths) != L:
        raise ValueError(f"lengths sum to {sum(lengths)}, not L={L}")
    return np.asarray(lengths, dtype=np.int64)


def cu_seqlens(lengths) -> np.ndarray:
    """Prefix sums [0, l0, l0+l1, ...] as int32."""
    lengths = np.asarray(lengths, dtype=np.int64)
    cu = np.zeros(len(lengths) + 1, dtype=np.int64)
    np.cumsum(lengths, out=cu[1:])
    if cu[-1] > np.iinfo(np.int32).max:
        raise ValueError("pack too long for int32 cu_seqlens")
    return cu.astype(np.int32)


def _fill_chunk(out: np.ndarray, seed: int, tid: int, c: int) -> None:
    lo = c * CHUNK
    hi = min(out.size, lo + CHUNK)
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(entropy=seed, spawn_key=(tid, c))))
    x = g.standard_normal(hi - lo, dtype=np.float32).view(np.uint32)
    x += ((x >> 16) & 1) + 0x7FFF          # round to nearest even on the 16 dropped bits
    out[lo:hi] = x >> 16


def bf16_normal(shape, seed: int, tensor: str, threads: int = None) -> np.ndarray:
    """N(0, 1) rounded to bf16, returned as uint16 bit patterns of the given shape."""
    tid = TENSOR_IDS[tensor]
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    nchunks = (n + CHUNK - 1) // CHUNK
    threads = threads or min(16, len(os.sched_getaffinity(0)))
    if nchunks == 1 or threads == 1:
        for c in range(nchunks):
            _fill_chunk(out, seed, tid, c)
    else:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(lambda c: _fill_chunk(out, seed, tid, c), range(nchunks)))
    return out.reshape(shape)


def make_tensors(w: Workload, seed: int, names=("q", "k", "v")) -> dict:
    """q [L, h_q, d], k/v [L, h_kv, d], dout [L, h_q, d] as bf16 bit patterns."""
    L, d = w.total_tokens, w.head_dim
    shapes = {"q": (L, w.h_q, d), "k": (L, w.h_kv, d), "v": (L, w.h_kv, d), "dout": (L, w.h_q, d)}
    return {n: bf16_normal(shapes[n], seed, n) for n in names}


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest even) and return the bit patterns."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).copy()
    b += ((b >> 16) & 1) + 0x7FFF
    return (b >> 16).astype(np.uint16)


def extreme_logit_inputs(w: Workload, cu, kind: str, seed: int, names=("q", "k", "v")) -> dict:
    """Seeded inputs whose scaled logits leave the N(0, 1) range (the bf16 bits are what both the
    GPU and the oracle read, so any transformation before rounding is exact for both):
      x4 / x8   q and k multiplied by 4 or 8 (powers of two: exact), logit std about 23 or 92 in
                log2 units, so block maxima jump by far more than the forward's rescale slack;
      rising    q ~ u and key j of a sample ~ a_j u with a_j growing 0.75 per 64 keys, so every key
                block's logits exceed all earlier ones by about 12 (log2 units): a rescale per block;
      falling   the same with a_j shrinking along the sample: later blocks sit far below the first
                maximum and their weights underflow."""
    t = make_tensors(w, seed, names=names)
    q = bf16_bits_to_f32(t["q"])
    k = bf16_bits_to_f32(t["k"])
    if kind in ("x4", "x8"):
        m = 4.0 if kind == "x4" else 8.0
        q, k = q * m, k * m
    elif kind in ("rising", "falling"):
        rng = np.random.default_rng(seed + 1000)
        u = rng.standard_normal(w.head_dim).astype(np.float32)
        lens = np.diff(cu)
        start = np.repeat(cu[:-1], lens)
        pos = (np.arange(w.total_tokens) - start).astype(np.float32)
        if kind == "falling":
            pos = np.repeat(lens, lens).astype(np.float32) - 1 - pos
        a = 0.75 * pos / 64.0
        k = a[:, None, None] * u[None, None, :] + 0.3 * k
        q = u[None, None, :] + 0.3 * q
    else:
        raise ValueError(kind)
    t["q"] = f32_to_bf16_bits(q.astype(np.float32))
    t["k"] = f32_to_bf16_bits(k.astype(np.float32))
    return t
