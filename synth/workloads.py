"""Seeded synthetic inputs for paged decode attention.

This module is the one piece of code that both the oracle and the GPU path
consume.  It holds no attention or allocation arithmetic: only workload shapes,
seeded random draws (context lengths, pool orders, q/K/V values, operation
scripts) and storage encodings (bf16 bits, fp16, fp32) with their exact
decoding to float64.

Workload shapes follow the decode scenarios the pages describe: fixed 16-token
KV blocks ("Stop Wasting GPU Memory" page, Technical Details, "Core
Architecture"; the ml-canon page's block-table box, block_size = 16), scattered
physical blocks, shared-prefix sampling with copy-on-write (same page,
"Copy-on-Write for Parallel Sampling") and 128K-token contexts (same page,
Industry Insight).

Every random draw comes from ``numpy.random.Generator(PCG64(SeedSequence(
[cfg_id, purpose, *index])))`` so any one sequence or head can be regenerated
on its own.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

# purpose codes of the seed streams
P_LENS, P_POOL, P_Q, P_K, P_V, P_KNEW, P_VNEW, P_MISC = 1, 2, 3, 4, 5, 6, 7, 8

DTYPES = ("f32", "bf16", "f16")
ELEM_BYTES = {"f32": 4, "bf16": 2, "f16": 2}


def rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(key))))


# ---------------------------------------------------------------- encodings
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    Returns the 16-bit patterns as uint16.  NaN maps to the quiet NaN 0x7FC0.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    # uint32 arithmetic wraps only for patterns above 0xFFFF8000, which are NaNs
    # and are overwritten below.
    out = (u >> 16) & np.uint32(1)
    out += np.uint32(0x7FFF)
    out += u
    out >>= np.uint32(16)
    out = out.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def encode(x32: np.ndarray, dtype: str) -> np.ndarray:
    """Store float32 values in ``dtype``: f32 as is, f16 by numpy's RNE cast,
    bf16 as uint16 bit patterns (RNE)."""
    if dtype == "f32":
        return np.ascontiguousarray(x32, dtype=np.float32)
    if dtype == "f16":
        return x32.astype(np.float16)
    if dtype == "bf16":
        return f32_to_bf16_bits(x32)
    raise ValueError(dtype)


def decode_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of stored elements (every f32/f16/bf16 value is
    representable in float64)."""
    if dtype == "bf16":
        return bf16_bits_to_f32(x).astype(np.float64)
    return np.asarray(x).astype(np.float64)


def storage_np_dtype(dtype: str):
    return {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}[dtype]


def nan_pattern(dtype: str):
    """Element value used to poison cache memory that must never be read."""
    if dtype == "bf16":
        return np.uint16(0x7FC0)
    return storage_np_dtype(dtype)(np.nan)


# ---------------------------------------------------------------- configs
@dataclass(frozen=True)
class DecodeConfig:
    """One decode-attention workload (one layer)."""

    name: str
    cfg_id: int
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    dtype: str
    lens: str                      # "fixed" | "uniform" | "lognormal"
    lens_args: tuple = ()
    block_size: int = 16
    scale: float = 0.0             # 0 -> 1/sqrt(head_dim)
    partition_size: int = 512
    preoccupied_frac: float = 0.0  # fraction of the pool held by a foreign sequence
    pool_slack_tokens: int = 0     # room for later decode appends, per sequence
    description: str = ""

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def softmax_scale(self) -> float:
        s = self.scale if self.scale else 1.0 / math.sqrt(self.head_dim)
        return float(np.float32(s))

    @property
    def elem_bytes(self) -> int:
        return ELEM_BYTES[self.dtype]

    def kv_bytes_per_token(self) -> int:
        """K and V bytes of one token of one layer: 2 * n_kv_heads * d_head * elem."""
        return 2 * self.num_kv_heads * self.head_dim * self.elem_bytes


C1 = DecodeConfig("c1_tiny_f32", 1, 4, 4, 4, 64, "f32", "fixed", (1, 15, 16, 33),
                  scale=0.125,
                  description="tiny fp32 MHA decode, ctx {1,15,16,33}, 4 heads, D=64, 32-block pool")
C2 = DecodeConfig("c2_mha_bf16", 2, 64, 32, 32, 128, "bf16", "uniform", (128, 2048),
                  pool_slack_tokens=256,
                  description="bf16 MHA decode, 64 seqs, ctx U[128,2048], 32/32 heads, D=128")
C3 = DecodeConfig("c3_gqa_bf16", 3, 256, 64, 8, 128, "bf16", "lognormal", (1024.0, 1.0, 16, 8192),
                  preoccupied_frac=0.3, pool_slack_tokens=64,
                  description="bf16 GQA decode, 256 seqs, lognormal ctx (median 1024, sigma 1, "
                              "clip [16,8192]), 64/8 heads, D=128, 30% of pool pre-occupied")
C5 = DecodeConfig("c5_long_bf16", 5, 4, 64, 8, 128, "bf16", "fixed", (131072,) * 4,
                  pool_slack_tokens=64,
                  description="bf16 long-context GQA decode, 4 x 131072 tokens, 64/8 heads, D=128, "
                              "512-token partitions + reduce")

CONFIGS = {c.name: c for c in (C1, C2, C3, C5)}


def context_lens(cfg: DecodeConfig) -> np.ndarray:
    """Per-sequence context lengths (tokens already cached, including the
    current decode token)."""
    if cfg.lens == "fixed":
        out = np.asarray(cfg.lens_args, dtype=np.int64)
        assert out.size == cfg.num_seqs
    elif cfg.lens == "uniform":
        lo, hi = cfg.lens_args
        out = rng(cfg.cfg_id, P_LENS).integers(lo, hi, size=cfg.num_seqs, endpoint=True)
    elif cfg.lens == "lognormal":
        median, sigma, lo, hi = cfg.lens_args
        draw = rng(cfg.cfg_id, P_LENS).lognormal(math.log(median), sigma, size=cfg.num_seqs)
        out = np.clip(np.rint(draw), lo, hi)
    else:
        raise ValueError(cfg.lens)
    return out.astype(np.int32)


def blocks_for(n_tokens, block_size: int = 16):
    return -(-np.asarray(n_tokens, dtype=np.int64) // block_size)


@dataclass
class PoolPlan:
    num_blocks: int
    free_order: np.ndarray          # int32 permutation of [0, num_blocks): hand-out order
    preoccupy_blocks: int           # blocks a foreign sequence takes before the workload


def pool_plan(cfg: DecodeConfig, lens: np.ndarray | None = None) -> PoolPlan:
    """Pool size and seeded hand-out order for a workload.

    The pool holds every sequence's blocks plus room for ``pool_slack_tokens``
    more tokens per sequence; with ``preoccupied_frac`` = f the pool is grown
    so that the workload's blocks are 1-f of it and a foreign sequence takes
    the first f of the shuffled hand-out order.
    """
    if lens is None:
        lens = context_lens(cfg)
    need = int(blocks_for(np.asarray(lens) + cfg.pool_slack_tokens, cfg.block_size).sum())
    if cfg.name == C1.name:
        n = 32
    elif cfg.preoccupied_frac > 0:
        n = int(math.ceil(need / (1.0 - cfg.preoccupied_frac)))
    else:
        n = need
    order = rng(cfg.cfg_id, P_POOL).permutation(n).astype(np.int32)
    pre = int(round(cfg.preoccupied_frac * n))
    return PoolPlan(n, order, pre)


def seq_kv(cfg: DecodeConfig, s: int, ctx: int, kv_heads=None):
    """K and V of sequence ``s`` for positions [0, ctx): arrays [ctx, H_kv, D]
    in storage encoding.  Head h of sequence s has its own seed stream, so a
    subset of heads can be drawn alone (``kv_heads``)."""
    heads = range(cfg.num_kv_heads) if kv_heads is None else kv_heads
    ks, vs = [], []
    for h in heads:
        ks.append(rng(cfg.cfg_id, P_K, s, h).standard_normal((ctx, cfg.head_dim), dtype=np.float32))
        vs.append(rng(cfg.cfg_id, P_V, s, h).standard_normal((ctx, cfg.head_dim), dtype=np.float32))
    k = np.stack(ks, axis=1) if ks else np.zeros((ctx, 0, cfg.head_dim), np.float32)
    v = np.stack(vs, axis=1) if vs else np.zeros((ctx, 0, cfg.head_dim), np.float32)
    return encode(k, cfg.dtype), encode(v, cfg.dtype)


def queries(cfg: DecodeConfig, step: int = 0, num_seqs: int | None = None) -> np.ndarray:
    """Decode queries [S, H_q, D] in storage encoding."""
    n = cfg.num_seqs if num_seqs is None else num_seqs
    q = rng(cfg.cfg_id, P_Q, step).standard_normal((n, cfg.num_q_heads, cfg.head_dim), dtype=np.float32)
    return encode(q, cfg.dtype)


def new_tokens_kv(cfg_id: int, step: int, num_tokens: int, num_kv_heads: int, head_dim: int,
                  dtype: str):
    """K/V of tokens appended at decode step ``step``: [T, H_kv, D] each."""
    k = rng(cfg_id, P_KNEW, step).standard_normal((num_tokens, num_kv_heads, head_dim), dtype=np.float32)
    v = rng(cfg_id, P_VNEW, step).standard_normal((num_tokens, num_kv_heads, head_dim), dtype=np.float32)
    return encode(k, dtype), encode(v, dtype)


# ---------------------------------------------------------------- parallel sampling
@dataclass(frozen=True)
class SamplingConfig:
    """Parallel sampling over a shared prompt prefix (copy-on-write workload).

    ``num_prompts`` prompts of ``prefix_len`` tokens; each is forked into
    ``samples`` branches which then each append ``steps`` tokens, one per
    decode step.  Sequence id of prompt i, sample k is i * samples + k; sample
    0 is the prompt's own sequence and samples 1.. are forks of it.
    """

    name: str = "c4_cow_sampling_bf16"
    cfg_id: int = 4
    num_prompts: int = 64
    samples: int = 8
    prefix_len: int = 1000
    steps: int = 200
    num_q_heads: int = 32
    num_kv_heads: int = 8
    head_dim: int = 128
    dtype: str = "bf16"
    block_size: int = 16
    partition_size: int = 512
    slack_blocks: int = 256
    description: str = ("parallel sampling with copy-on-write: 64 prompts x 8 samples, shared "
                        "1000-token prefix, 200 appended tokens per sample, bf16 GQA 32/8, D=128")

    @property
    def num_seqs(self) -> int:
        return self.num_prompts * self.samples

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def softmax_scale(self) -> float:
        return float(np.float32(1.0 / math.sqrt(self.head_dim)))

    @property
    def elem_bytes(self) -> int:
        return ELEM_BYTES[self.dtype]

    def kv_bytes_per_token(self) -> int:
        return 2 * self.num_kv_heads * self.head_dim * self.elem_bytes

    def pool_blocks(self) -> int:
        b = self.block_size
        full_shared = self.prefix_len // b
        per_sample = -(-(self.prefix_len + self.steps) // b) - full_shared
        return self.num_prompts * (full_shared + self.samples * per_sample) + self.slack_blocks

    def free_order(self) -> np.ndarray:
        return rng(self.cfg_id, P_POOL).permutation(self.pool_blocks()).astype(np.int32)

    def prefix_kv(self, prompt: int, kv_heads=None):
        heads = range(self.num_kv_heads) if kv_heads is None else kv_heads
        ks = [rng(self.cfg_id, P_K, prompt, h).standard_normal((self.prefix_len, self.head_dim), dtype=np.float32)
              for h in heads]
        vs = [rng(self.cfg_id, P_V, prompt, h).standard_normal((self.prefix_len, self.head_dim), dtype=np.float32)
              for h in heads]
        return encode(np.stack(ks, axis=1), self.dtype), encode(np.stack(vs, axis=1), self.dtype)

    def step_kv(self, step: int):
        """K/V appended at decode step ``step`` (1-based): [num_seqs, H_kv, D]."""
        return new_tokens_kv(self.cfg_id, step, self.num_seqs, self.num_kv_heads, self.head_dim, self.dtype)

    def step_q(self, step: int):
        q = rng(self.cfg_id, P_Q, step).standard_normal(
            (self.num_seqs, self.num_q_heads, self.head_dim), dtype=np.float32)
        return encode(q, self.dtype)


C4 = SamplingConfig()


def scaled(cfg: DecodeConfig, num_seqs: int | None = None, lens=None, name_suffix="_small",
           **kw) -> DecodeConfig:
    """A smaller copy of a decode config with the same head layout, for
    parity runs the oracle finishes in seconds."""
    d = dict(cfg.__dict__)
    d.update(kw)
    d["name"] = cfg.name + name_suffix
    if num_seqs is not None:
        d["num_seqs"] = num_seqs
    if lens is not None:
        d["lens"] = "fixed"
        d["lens_args"] = tuple(int(x) for x in lens)
        d["num_seqs"] = len(lens)
    return DecodeConfig(**d)
