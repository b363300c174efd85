"""Seeded synthetic inputs for the paged decode workloads.

This module only draws random numbers: sequence lengths, the initial order of the
free-block queue, token K/V/q values and the churn events. It holds none of the
method's arithmetic (no slot or block-table computation, no attention), so the CPU
oracle and the HIP path can both take their inputs from it without sharing code.

Every draw goes through ``numpy.random.Generator(PCG64(seed))``; floating-point
values are drawn in float32 and cast to the workload dtype with round-to-nearest-
even, and the cast bits are the true input for both sides.

Workload shapes (model shapes and length mixes) follow the pages:
  * Llama-3-70B: 80 layers, 64 attention heads, 8 KV heads, head_dim 128, FP16
    ("Yerel LLM sistemlerinde backpressure ve ölçekleme", section "KV bütçesi").
  * a 32-layer GQA model with 8 KV heads, head_dim 128, bf16
    ("vLLM Nedir? PagedAttention ile Production LLM Serving", section
    "Asıl şişen şey ağırlık değil, KV cache").
  * the short/long request mix 300/100 and 30,000/4,000 tokens
    ("Yerel LLM ...", section "Her istek eşit değildir").
  * a shared 1,000-2,000-token system prompt (same page, section "4. Prefill ve decode",
    paragraph on prefix caching).
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

BLOCK_SIZE = 16

# dtype name -> (bytes per element, numpy storage dtype of the raw bits)
DTYPES = {"f32": (4, np.uint32), "f16": (2, np.uint16), "bf16": (2, np.uint16)}


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    layers: int
    batch: int
    num_heads: int
    num_kv_heads: int
    head_dim: int
    dtype: str
    seed: int
    kv_std: float = 1.0
    q_std: float = 1.0
    len_lo: int = 0
    len_hi: int = 0
    # two-class length mix (short/long); used when long_frac > 0
    long_frac: float = 0.0
    long_lo: int = 0
    long_hi: int = 0
    # decode launch: 0 one pass per (sequence, KV head), > 0 fixed context partitions of
    # that many tokens, -1 the balanced split
    partition_size: int = 0
    num_blocks: int = 0          # 0: sized from the drawn lengths
    # churn
    pool_bytes: float = 0.0
    retire_frac: float = 0.0
    share_frac: float = 0.0
    prefix_tokens: int = 0
    prompt_lo: int = 0
    prompt_hi: int = 0
    # chunked prefill: a prefill_tokens-token prompt in prefill_chunks chunks, each step also
    # decoding one token for each of `batch` users
    prefill_tokens: int = 0
    prefill_chunks: int = 0
    # tokens per KV block (16; 8 and 32 are the block-size variants)
    block_size: int = 16
    # KV cache element type ("" = dtype; "fp8" = OCP e4m3 codes of x / k_scale, x / v_scale)
    kv_dtype: str = ""
    k_scale: float = 1.0
    v_scale: float = 1.0

    @property
    def group(self) -> int:
        return self.num_heads // self.num_kv_heads

    @property
    def cache_dtype(self) -> str:
        return self.kv_dtype or self.dtype

    @property
    def cache_elem_bytes(self) -> int:
        return 1 if self.cache_dtype == "fp8" else self.elem_bytes

    @property
    def elem_bytes(self) -> int:
        return DTYPES[self.dtype][0]

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def block_bytes_per_layer(self) -> int:
        """Bytes of one physical block (K and V, all KV heads) in one layer."""
        return 2 * self.num_kv_heads * self.block_size * self.head_dim * self.cache_elem_bytes


WORKLOADS = {
    # 1 layer, B 4, 8q/2kv, d 64, fp32, n ~ U{1..256}, 128-block pool.
    "tiny": Workload("tiny", layers=1, batch=4, num_heads=8, num_kv_heads=2, head_dim=64,
                     dtype="f32", seed=28001, len_lo=1, len_hi=256, num_blocks=128),
    # Llama-3-8B shape: 32 layers, 32q/8kv, d 128, bf16, B 64, n ~ U{128..2048}.
    "llama8b": Workload("llama8b", layers=32, batch=64, num_heads=32, num_kv_heads=8,
                        head_dim=128, dtype="bf16", seed=28002, len_lo=128, len_hi=2048,
                        partition_size=0),
    # The same with an FP8 (e4m3) KV cache: per-tensor scales put N(0,1) rows at up to
    # about 6.7 (K) and 5.6 (V) standard deviations inside e4m3's +-448.
    "llama8b_fp8": Workload("llama8b_fp8", layers=32, batch=64, num_heads=32, num_kv_heads=8,
                            head_dim=128, dtype="bf16", seed=28002, len_lo=128, len_hi=2048,
                            partition_size=0, kv_dtype="fp8", k_scale=0.015, v_scale=0.0125),
    # Llama-3-70B shape: 80 layers, 64q/8kv, d 128, fp16, B 128; 90% short
    # (300 prompt + up to 100 generated), 10% long (30,000 + up to 4,000). The ragged mix
    # runs best in the balanced split.
    "llama70b": Workload("llama70b", layers=80, batch=128, num_heads=64, num_kv_heads=8,
                         head_dim=128, dtype="f16", seed=28003, len_lo=300, len_hi=400,
                         long_frac=0.1, long_lo=30000, long_hi=34000, partition_size=-1),
    # Long-context split-K: 1 layer, B 4, 32q/8kv, bf16, n ~ U{131072..262144},
    # 512-token partitions, K/V ~ N(0, 0.5^2).
    "long": Workload("long", layers=1, batch=4, num_heads=32, num_kv_heads=8, head_dim=128,
                     dtype="bf16", seed=28004, kv_std=0.5, len_lo=131072, len_hi=262144,
                     partition_size=512),
    # Chunked prefill ("Yerel LLM ...", section "4. Prefill ve decode": a 30,000-token
    # document summary arriving among 20 streaming users; chunked, each step computes one
    # prefill chunk and one decode token per user, 1/8 of the prompt per step in the
    # page's diagram), on the 8B shape; the users' contexts as in the 8B workload.
    "prefill_30k": Workload("prefill_30k", layers=32, batch=20, num_heads=32, num_kv_heads=8,
                            head_dim=128, dtype="bf16", seed=28006, len_lo=128, len_hi=2048,
                            prefill_tokens=30000, prefill_chunks=8),
    # Continuous-batching churn on the 8B shape with a ~200 GB pool.
    "churn": Workload("churn", layers=32, batch=256, num_heads=32, num_kv_heads=8,
                      head_dim=128, dtype="bf16", seed=28005, pool_bytes=200e9,
                      retire_frac=0.05, share_frac=0.2, prefix_tokens=1024,
                      prompt_lo=16, prompt_hi=32768, partition_size=-1),
}


def rng(seed: int, *stream: int) -> np.random.Generator:
    """Independent generator for (seed, stream...) so each layer/step draws its own data."""
    return np.random.Generator(np.random.PCG64([seed, *stream]))


def draw_seq_lens(w: Workload, gen: np.random.Generator | None = None) -> np.ndarray:
    """Context lengths n_b (inclusive of the token being decoded), int64 [batch]."""
    gen = gen or rng(w.seed, 0)
    if w.long_frac > 0:
        n_long = int(round(w.long_frac * w.batch))
        lens = np.concatenate([
            gen.integers(w.long_lo, w.long_hi, size=n_long, endpoint=True),
            gen.integers(w.len_lo, w.len_hi, size=w.batch - n_long, endpoint=True)])
        gen.shuffle(lens)
        return lens.astype(np.int64)
    return gen.integers(w.len_lo, w.len_hi, size=w.batch, endpoint=True).astype(np.int64)


def draw_free_order(num_blocks: int, gen: np.random.Generator) -> np.ndarray:
    """A random permutation of 0..num_blocks-1: the initial free-queue order, which
    scatters every sequence's blocks over the pool."""
    return gen.permutation(num_blocks).astype(np.int32)


def _cast(x32: np.ndarray, dtype: str):
    """float32 array -> torch tensor in the workload dtype (round to nearest even)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x32))
    return t.to({"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dtype])


def draw_tokens(n_tokens: int, w: Workload, gen: np.random.Generator, std: float | None = None):
    """K or V rows for n_tokens tokens: torch [n_tokens, num_kv_heads, head_dim] on CPU."""
    std = w.kv_std if std is None else std
    x = gen.standard_normal((n_tokens, w.num_kv_heads, w.head_dim), dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return _cast(x, w.dtype)


def draw_q(w: Workload, gen: np.random.Generator, batch: int | None = None):
    """Queries: torch [batch, num_heads, head_dim] on CPU."""
    b = w.batch if batch is None else batch
    x = gen.standard_normal((b, w.num_heads, w.head_dim), dtype=np.float32)
    if w.q_std != 1.0:
        x *= np.float32(w.q_std)
    return _cast(x, w.dtype)


def _torch_seed(seed: int, stream) -> int:
    """A 63-bit seed for torch's generator derived from (seed, *stream) via PCG64."""
    return int(rng(seed, *stream).integers(0, 2 ** 63 - 1))


def draw_tokens_device(n_tokens: int, w: Workload, stream, device, std: float | None = None):
    """K or V rows [n_tokens, num_kv_heads, head_dim] drawn directly on a device with a
    torch generator seeded from (w.seed, *stream); for the multi-GB workloads. The same
    (seed, stream, device type) always gives the same values."""
    import torch
    std = w.kv_std if std is None else std
    g = torch.Generator(device=device)
    g.manual_seed(_torch_seed(w.seed, tuple(stream)))
    x = torch.randn((n_tokens, w.num_kv_heads, w.head_dim), generator=g, device=device,
                    dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x.to({"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[w.dtype])


def draw_q_device(w: Workload, stream, device, batch: int | None = None):
    """Queries [batch, num_heads, head_dim] drawn on a device (see draw_tokens_device)."""
    import torch
    b = w.batch if batch is None else batch
    g = torch.Generator(device=device)
    g.manual_seed(_torch_seed(w.seed, tuple(stream)))
    x = torch.randn((b, w.num_heads, w.head_dim), generator=g, device=device,
                    dtype=torch.float32)
    if w.q_std != 1.0:
        x.mul_(w.q_std)
    return x.to({"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[w.dtype])


def pool_blocks_for(lens, growth_tokens: int = 0, slack: float = 0.10,
                    block_size: int = BLOCK_SIZE) -> int:
    """Pool size (blocks) that holds every sequence plus growth_tokens more each,
    plus a slack fraction of unused blocks."""
    need = sum(-(-(int(n) + growth_tokens) // block_size) for n in lens)
    return int(need * (1.0 + slack)) + 1


# ---------------------------------------------------------------- churn events
def churn_pool_blocks(w: Workload) -> int:
    """floor(pool_bytes / (layers * bytes of one block per layer))."""
    return int(w.pool_bytes // (w.layers * w.block_bytes_per_layer))


def draw_prompt_len(w: Workload, gen: np.random.Generator) -> int:
    """Log-uniform prompt length in [prompt_lo, prompt_hi]."""
    u = gen.uniform(math.log(w.prompt_lo), math.log(w.prompt_hi))
    return int(min(w.prompt_hi, max(w.prompt_lo, math.floor(math.exp(u)))))


def draw_churn_initial(w: Workload, gen: np.random.Generator):
    """Initial batch: list of (is_sharer, own_prompt_len). Exactly round(share_frac*B)
    sequences share the prefix."""
    n_share = int(round(w.share_frac * w.batch))
    sharer = np.zeros(w.batch, dtype=bool)
    sharer[gen.choice(w.batch, size=n_share, replace=False)] = True
    return [(bool(s), draw_prompt_len(w, gen)) for s in sharer]


def draw_churn_step(w: Workload, gen: np.random.Generator, live_ids):
    """One churn step: which live sequences retire (positions into live_ids) and the
    (is_sharer, own_prompt_len) of each admitted sequence."""
    n = int(round(w.retire_frac * len(live_ids)))
    retire = sorted(gen.choice(len(live_ids), size=n, replace=False).tolist())
    admits = [(bool(gen.random() < w.share_frac), draw_prompt_len(w, gen)) for _ in range(n)]
    return retire, admits
