"""Seeded synthetic workloads: shapes, distributions and generators only.

This module holds none of the attention arithmetic.  It is the one piece the
HIP path's tests/bench and the CPU oracle share: both read the same host
arrays drawn here.  Shapes follow the workloads the pages describe
(Whisper-encoder-shaped multi-head attention; Llama-style GQA decode against
a batched cache of up to 32 sequences -- realizar 0.8.5
``src/cuda/executor/cache_from_cache_from_kv_cache.rs``,
``init_batched_kv_cache_gpu``).  No dataset is involved: every tensor is
``numpy.random.default_rng(1000 + config_id).standard_normal(..., float32)``
times a fixed factor, drawn in a fixed order (prefill: Q, K, V; decode: lengths,
q, k_new, v_new, K cache, V cache).
"""
from __future__ import annotations

import dataclasses

import numpy as np

# Quiet-NaN bit pattern used to fill cache regions that no step defines, so a
# stray read or write shows up in a bit-exact comparison.
SENTINEL_BITS = 0x7FC0DEAD


def scale_for(d: int) -> float:
    """1.0f / sqrtf(d), the f32 value passed to both the GPU path and the oracle."""
    return float(np.float32(1.0) / np.sqrt(np.float32(d)))


@dataclasses.dataclass(frozen=True)
class PrefillConfig:
    cid: int
    name: str
    B: int
    S: int
    H: int
    d: int
    causal: bool
    std: float = 1.0

    @property
    def scale(self) -> float:
        return scale_for(self.d)

    @property
    def visible_pairs(self) -> int:
        """Query/key pairs that enter a softmax (masked pairs excluded)."""
        per_head = self.S * (self.S + 1) // 2 if self.causal else self.S * self.S
        return self.B * self.H * per_head

    @property
    def flops(self) -> int:
        """2*d for Q.K plus 2*d for P.V per visible pair."""
        return 4 * self.d * self.visible_pairs

    @property
    def io_bytes(self) -> int:
        """Q, K, V read once and O written once."""
        return 4 * 4 * self.B * self.S * self.H * self.d


@dataclasses.dataclass(frozen=True)
class DecodeConfig:
    cid: int
    name: str
    M: int
    H: int
    Hkv: int
    d: int
    max_len: int
    len_lo: int
    len_hi: int

    @property
    def scale(self) -> float:
        return scale_for(self.d)

    def decode_bytes(self, lens) -> int:
        """K and V rows 0..L_m-1 of every KV head, plus q read and out written."""
        total = int(np.sum(np.asarray(lens, dtype=np.int64)))
        return 2 * self.Hkv * self.d * 4 * total + 2 * self.M * self.H * self.d * 4

    def decode_flops(self, lens) -> int:
        total = int(np.sum(np.asarray(lens, dtype=np.int64)))
        return 4 * self.d * self.H * total

    @property
    def append_bytes(self) -> int:
        """One new K and V row per sequence: read once, written once."""
        return 2 * 2 * self.M * self.Hkv * self.d * 4


@dataclasses.dataclass(frozen=True)
class ScatterConfig:
    cid: int
    name: str
    M: int
    n_new: int
    Hkv: int
    d: int
    max_len: int

    @property
    def bytes(self) -> int:
        """K and V sources read once, cache rows written once."""
        return 2 * 2 * self.M * self.n_new * self.Hkv * self.d * 4


@dataclasses.dataclass(frozen=True)
class ChunkConfig:
    """A chunk of n_new tokens prefilled behind cached[m] rows of each sequence."""
    name: str
    M: int
    n_new: int
    H: int
    Hkv: int
    d: int
    max_len: int

    @property
    def scale(self) -> float:
        return scale_for(self.d)

    def flops(self, cached) -> int:
        """4*d per visible (query, key) pair per head: query r of sequence m sees cached[m] + r + 1 keys."""
        pairs = sum(int(c) * self.n_new + self.n_new * (self.n_new + 1) // 2 for c in cached)
        return 4 * self.d * self.H * pairs


PREFILL = {
    1: PrefillConfig(1, "mha_s64_h4_d32", B=1, S=64, H=4, d=32, causal=False),
    2: PrefillConfig(2, "whisper_base_encoder_s1500_h8_d64", B=1, S=1500, H=8, d=64, causal=False),
    3: PrefillConfig(3, "causal_b4_s2048_h32_d128", B=4, S=2048, H=32, d=128, causal=True, std=0.5),
}
# The bulk append of the causal prefill's K/V into a [4, 32, 4096, 128] cache from position 0.
BULK_SCATTER = ScatterConfig(3, "bulk_append_m4_n2048_hkv32_d128_max4096", M=4, n_new=2048, Hkv=32,
                             d=128, max_len=4096)
# The second half of the causal prefill workload's sequences prefilled behind the first half.
CHUNK_BEHIND_CACHE = ChunkConfig("chunk_m4_n2048_behind_2048_h32_d128_max4096", M=4, n_new=2048, H=32, Hkv=32,
                                 d=128, max_len=4096)
DECODE = {
    4: DecodeConfig(4, "gqa_decode_m32_h32_hkv8_d128_max4096", M=32, H=32, Hkv=8, d=128,
                    max_len=4096, len_lo=1, len_hi=4096),
    5: DecodeConfig(5, "gqa_decode_m16_h64_hkv8_d128_max32768", M=16, H=64, Hkv=8, d=128,
                    max_len=32768, len_lo=16384, len_hi=32768),
}


def rng_for(cid: int) -> np.random.Generator:
    return np.random.default_rng(1000 + cid)


def normal(rng: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    a = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


def prefill_inputs(cfg: PrefillConfig, rng: np.random.Generator | None = None):
    """Q, K, V as [B, S, H*d] f32 (drawn in that order)."""
    rng = rng if rng is not None else rng_for(cfg.cid)
    shape = (cfg.B, cfg.S, cfg.H * cfg.d)
    q = normal(rng, shape, cfg.std)
    k = normal(rng, shape, cfg.std)
    v = normal(rng, shape, cfg.std)
    return q, k, v


def sentinel_cache(shape) -> np.ndarray:
    return np.full(shape, SENTINEL_BITS, dtype=np.uint32).view(np.float32)


def decode_inputs(cfg: DecodeConfig, rng: np.random.Generator | None = None,
                  fill_caches: bool = True):
    """One decode step's inputs.

    lens[m] ~ U{len_lo..len_hi} is the attention length after the append; the
    new row goes to position lens[m] - 1.  Returns a dict with lens (int32 [M]),
    q [M, H*d], k_new / v_new [M, 1, Hkv*d], k_cache / v_cache
    [M, Hkv, max_len, d] (N(0,1) when ``fill_caches``, else None).
    """
    rng = rng if rng is not None else rng_for(cfg.cid)
    lens = rng.integers(cfg.len_lo, cfg.len_hi + 1, size=cfg.M).astype(np.int32)
    q = normal(rng, (cfg.M, cfg.H * cfg.d))
    k_new = normal(rng, (cfg.M, 1, cfg.Hkv * cfg.d))
    v_new = normal(rng, (cfg.M, 1, cfg.Hkv * cfg.d))
    k_cache = v_cache = None
    if fill_caches:
        shape = (cfg.M, cfg.Hkv, cfg.max_len, cfg.d)
        k_cache = normal(rng, shape)
        v_cache = normal(rng, shape)
    return dict(lens=lens, q=q, k_new=k_new, v_new=v_new, k_cache=k_cache, v_cache=v_cache)
