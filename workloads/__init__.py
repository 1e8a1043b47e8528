"""Seeded synthetic inputs shaped like the pages' workloads.

This module only draws random tensors; it holds none of the codec's
arithmetic and is shared by the tests, the bench and the oracle checks.  The
pages measure on real models and datasets (LLM text, video and audio KV
caches) that are not available, so these seeded inputs stand in for them with
the same head dims, head counts, cache lengths and value distributions:

  1 toy          d=128, b=3, 1 head, 4096 fp32 N(0,1) keys, 1 fp32 query (logits)
  2 llm_decode   d=128, b=4, B=1, 32 query / 8 KV heads, 32768 keys per KV head,
                 bf16 N(0,1) keys with 4 fixed outlier channels x10, bf16 V,
                 1 bf16 query token (fused attention)
  3 extreme      d=128, b=2, B=4, 32/8 heads, 131072 keys per KV head, bf16
                 Student-t(5) entries rescaled per token to a LogNormal(0, 0.5)
                 norm, bf16 V (fused attention)
  4 video_block  d=64, b=3, 24 heads (no GQA), a 16384-key chunk encoded at cache
                 positions 49152..65535 of a 65536-key cache, 256 bf16 queries
                 per head (multi-query attention)
  5 qjl          d=128, b=3 + QJL, B=8, 32/8 heads, 65536 bf16 N(0,1) keys per
                 KV head, 1 bf16 query token (QJL logits)
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import torch


@dataclass(frozen=True)
class Config:
    cid: int
    name: str
    d: int
    b: int
    B: int
    Hq: int
    Hkv: int
    N: int              # cached keys per KV head
    kdtype: str         # "f32" | "bf16"
    qdtype: str
    n_q: int            # query tokens per head
    mode: str           # "logits" | "attn" | "attn_mq"
    keys: str           # "gauss" | "outliers" | "student_t"
    qjl: bool = False
    chunk: int = 0      # encoded chunk (video block) placed at the end of the cache

    @property
    def n_seq(self) -> int:
        return self.B * self.Hkv

    @property
    def cap(self) -> int:
        return ((self.N + 63) // 64) * 64

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    def scaled(self, **kw) -> "Config":
        return replace(self, **kw)


CONFIGS = {
    1: Config(1, "toy", 128, 3, 1, 1, 1, 4096, "f32", "f32", 1, "logits", "gauss"),
    2: Config(2, "llm_decode", 128, 4, 1, 32, 8, 32768, "bf16", "bf16", 1, "attn", "outliers"),
    3: Config(3, "extreme", 128, 2, 4, 32, 8, 131072, "bf16", "bf16", 1, "attn", "student_t"),
    4: Config(4, "video_block", 64, 3, 1, 24, 24, 65536, "bf16", "bf16", 256, "attn_mq", "gauss",
              chunk=16384),
    5: Config(5, "qjl", 128, 3, 8, 32, 8, 65536, "bf16", "bf16", 1, "logits", "gauss", qjl=True),
}
# the same workloads by name
WORKLOADS = {c.name: c for c in CONFIGS.values()}

_DT = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def _gen(device, seed: int, stream: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed * 1_000_003 + stream)
    return g


def outlier_channels(cfg: Config, seed: int = 0):
    """The 4 fixed outlier channels of the LLM-decode keys (drawn once)."""
    g = _gen("cpu", seed, 4)
    return torch.randperm(cfg.d, generator=g)[:4]


def make_keys(cfg: Config, device="cpu", seed: int = 0, n_seq: int | None = None,
              n: int | None = None, stream: int = 1) -> torch.Tensor:
    """Keys [n_seq, n, d] in the config's key dtype."""
    n_seq = cfg.n_seq if n_seq is None else n_seq
    n = cfg.N if n is None else n
    g = _gen(device, seed, stream)
    out = torch.empty((n_seq, n, cfg.d), dtype=_DT[cfg.kdtype], device=device)
    chunk = max(1, (1 << 25) // max(1, n * cfg.d))
    for s0 in range(0, n_seq, chunk):
        s1 = min(n_seq, s0 + chunk)
        shape = (s1 - s0, n, cfg.d)
        if cfg.keys == "student_t":
            z = torch.randn(shape, generator=g, device=device)
            chi2 = torch.zeros(shape, device=device)
            for _ in range(5):
                chi2 += torch.randn(shape, generator=g, device=device) ** 2
            t = z / torch.sqrt(chi2 / 5.0)
            norm = torch.exp(0.5 * torch.randn(shape[:2] + (1,), generator=g, device=device))
            x = t / torch.linalg.vector_norm(t, dim=-1, keepdim=True) * norm
        else:
            x = torch.randn(shape, generator=g, device=device)
            if cfg.keys == "outliers":
                x[..., outlier_channels(cfg, seed).to(device)] *= 10.0
        out[s0:s1] = x.to(out.dtype)
    return out


def make_values(cfg: Config, device="cpu", seed: int = 0, n_seq: int | None = None,
                cap: int | None = None) -> torch.Tensor:
    """Values [n_seq, cap, d] bf16 N(0,1) (uncompressed)."""
    n_seq = cfg.n_seq if n_seq is None else n_seq
    cap = cfg.cap if cap is None else cap
    g = _gen(device, seed, 2)
    out = torch.empty((n_seq, cap, cfg.d), dtype=torch.bfloat16, device=device)
    chunk = max(1, (1 << 25) // max(1, cap * cfg.d))
    for s0 in range(0, n_seq, chunk):
        s1 = min(n_seq, s0 + chunk)
        out[s0:s1] = torch.randn((s1 - s0, cap, cfg.d), generator=g, device=device).to(torch.bfloat16)
    return out


def make_queries(cfg: Config, device="cpu", seed: int = 0, B: int | None = None) -> torch.Tensor:
    """Queries [B, Hq, n_q, d] in the config's query dtype, N(0,1)."""
    B = cfg.B if B is None else B
    g = _gen(device, seed, 3)
    q = torch.randn((B, cfg.Hq, cfg.n_q, cfg.d), generator=g, device=device)
    return q.to(_DT[cfg.qdtype])


def make_quality_inputs(device="cpu", seed: int = 0, d: int = 128, n_keys: int = 1024,
                        n_queries: int = 16, n_distractors: int = 2048):
    """Inputs of the pages' synthetic quality experiment: isotropic Gaussian
    fp32 keys [1, n_keys, d] and queries [1, n_queries, d]; and a needle set,
    n_distractors Gaussian keys with one more key (the needle) at a seeded
    position, [1, n_distractors + 1, d], whose query is the needle itself.
    Returns (keys, queries, needle_keys, needle_query [1, 1, d], needle_pos)."""
    g = _gen(device, seed, 5)
    keys = torch.randn((1, n_keys, d), generator=g, device=device)
    queries = torch.randn((1, n_queries, d), generator=g, device=device)
    needle_keys = torch.randn((1, n_distractors + 1, d), generator=g, device=device)
    pos = int(torch.randint(0, n_distractors + 1, (1,), generator=g, device=device).item())
    needle_query = needle_keys[:, pos:pos + 1].clone()
    return keys, queries, needle_keys, needle_query, pos
