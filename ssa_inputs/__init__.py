"""Seeded synthetic inputs for the SSA dual-stream attention forward.

This module is the only code that both the fp64 oracle (via the tests) and the
HIP path (via the tests and the benchmark) consume. It draws random tensors and
nothing else: it holds none of the attention, pooling, selection or loss
arithmetic.

Recipe (one independent stream per (tensor, batch, head), so any head can be
regenerated alone and generation is parallel and thread-count independent):

* stream = ``torch.Generator`` (CPU, Mersenne twister) seeded with a fixed
  mix of ``(config seed, tensor id, batch, head)``; tensor ids 0 = Q, 1 = K,
  2 = V, 3 = planted structure.
* entries are ``torch.randn`` float32 (iid N(0, 1));
* "peaked" configurations plant structure per (batch, kv head): a unit
  direction ``u`` (float64 normal, normalised) and ``round(0.1 * n_blocks)``
  key blocks chosen without replacement; every token of a planted key block
  gets ``+2.0 * u`` and every query row of the q heads that read that kv head
  gets ``+2.0 * u`` (so the mean-pooled block similarity singles out the
  planted blocks and the softmax mass concentrates there);
* bf16 configurations round the float32 values to bfloat16 (round to nearest
  even) as the last step;
* backward inputs: the upstream gradients of the two attention outputs
  (tensor ids 4 = d_full, 5 = d_sparse) are iid N(0, 1) per (batch, q head),
  rounded the same way. The backward is linear in them, so their scale
  (1/n-sized alignment seeds in training) does not change relative errors.

The attention logit scale 1/sqrt(D) is applied inside the attention, not to
the entries.
"""
from __future__ import annotations

import dataclasses
import math
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, Optional, Tuple

import torch

T_Q, T_K, T_V, T_PLANT, T_DFULL, T_DSPARSE = 0, 1, 2, 3, 4, 5
_MASK63 = (1 << 63) - 1


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    dtype: str            # "f32" or "bf16"
    B: int
    Hq: int
    Hkv: int
    N: int                # prefill: sequence length; decode: KV length
    D: int
    block: int
    budget: int           # total selected blocks per row, forced ones included
    n_sink: int
    n_local: int
    decode: bool
    planted: bool
    seed: int
    budgets: Tuple[int, ...] = ()

    @property
    def Nq(self) -> int:
        return 1 if self.decode else self.N

    @property
    def n_blocks(self) -> int:
        return self.N // self.block

    def with_budget(self, budget: int) -> "Config":
        return dataclasses.replace(self, budget=budget)

    def with_sizes(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)


# The workloads. Sink = first block, local = the block holding the
# query (the diagonal block in prefill, the most recent block in decode).
CONFIGS: Dict[str, Config] = {
    "tiny_f32": Config("tiny_f32", "f32", 1, 1, 1, 512, 64, 64, 4, 1, 1,
                       False, False, 0),
    "mha_4k": Config("mha_4k", "bf16", 1, 8, 8, 4096, 128, 64, 16, 1, 1,
                     False, False, 1),
    "gqa_8k_peaked": Config("gqa_8k_peaked", "bf16", 4, 32, 8, 8192, 128, 64,
                            16, 1, 1, False, True, 2),
    "gqa_32k_sweep": Config("gqa_32k_sweep", "bf16", 1, 32, 8, 32768, 128, 64,
                            16, 1, 1, False, True, 3, budgets=(4, 8, 16, 32)),
    "gqa_decode_64k": Config("gqa_decode_64k", "bf16", 64, 32, 8, 65536, 128,
                             64, 32, 1, 1, True, True, 4),
    # the pages' own model shape: 16-token blocks, 16 selected blocks (a
    # 256-token receptive field), head dim 64, 32 q heads over 2 kv heads
    "paper_16k_b16": Config("paper_16k_b16", "bf16", 1, 32, 2, 16384, 64, 16,
                            16, 1, 1, False, True, 5),
}
CONFIG_ORDER = ["tiny_f32", "mha_4k", "gqa_8k_peaked", "gqa_32k_sweep",
                "gqa_decode_64k", "paper_16k_b16"]


def stream_seed(seed: int, tensor_id: int, b: int, h: int) -> int:
    """Fixed mix of the four stream coordinates into a 63-bit seed."""
    x = 0x9E3779B97F4A7C15
    for v in (seed, tensor_id, b, h):
        x = ((x ^ (v + 0x632BE59BD9B4E019)) * 0xBF58476D1CE4E5B9) & _MASK63
        x ^= x >> 29
    return x & _MASK63


def _gen(seed: int, tensor_id: int, b: int, h: int) -> torch.Generator:
    return torch.Generator(device="cpu").manual_seed(stream_seed(seed, tensor_id, b, h))


def default_head_map(Hq: int, Hkv: int):
    g = Hq // Hkv
    return [h // g for h in range(Hq)]


def plant(cfg: Config, b: int, g: int) -> Tuple[torch.Tensor, torch.Tensor]:
    """Planted direction u [D] (float64, unit norm) and sorted planted key
    block ids for (batch b, kv head g)."""
    gen = _gen(cfg.seed, T_PLANT, b, g)
    u = torch.randn(cfg.D, generator=gen, dtype=torch.float64)
    u = u / torch.linalg.vector_norm(u)
    n_plant = int(round(0.1 * cfg.n_blocks))
    blocks = torch.randperm(cfg.n_blocks, generator=gen)[:n_plant]
    return u, torch.sort(blocks).values


def _slice(cfg: Config, tensor_id: int, b: int, h: int, rows: int,
           head_map) -> torch.Tensor:
    """One [rows, D] float32 slice of tensor `tensor_id` for (b, h)."""
    x = torch.randn(rows, cfg.D, generator=_gen(cfg.seed, tensor_id, b, h),
                    dtype=torch.float32)
    if cfg.planted and tensor_id in (T_Q, T_K):
        g = head_map[h] if tensor_id == T_Q else h
        u, blocks = plant(cfg, b, g)
        add = (2.0 * u).to(torch.float32)
        if tensor_id == T_Q:
            x += add
        else:
            bs = cfg.block
            for blk in blocks.tolist():
                x[blk * bs:(blk + 1) * bs] += add
    return x


def _fill(out: torch.Tensor, cfg: Config, tensor_id: int, rows: int,
          head_map, workers: int) -> None:
    B, H = out.shape[0], out.shape[1]

    def work(bh):
        b, h = divmod(bh, H)
        x = _slice(cfg, tensor_id, b, h, rows, head_map)
        out[b, h].copy_(x.to(out.dtype))

    if workers <= 1 or B * H == 1:
        for bh in range(B * H):
            work(bh)
    else:
        with ThreadPoolExecutor(max_workers=workers) as ex:
            list(ex.map(work, range(B * H)))


def torch_dtype(cfg: Config) -> torch.dtype:
    return torch.float32 if cfg.dtype == "f32" else torch.bfloat16


def make_inputs(cfg: Config, workers: int = 8, head_map=None,
                pin_memory: bool = False) -> Dict[str, torch.Tensor]:
    """Q [B,Hq,Nq,D], K and V [B,Hkv,N,D] as CPU tensors of the config dtype.

    Decode configurations give Q one row per (batch, q head): the query that
    sits at position N-1.
    """
    hm = head_map if head_map is not None else default_head_map(cfg.Hq, cfg.Hkv)
    dt = torch_dtype(cfg)
    q = torch.empty(cfg.B, cfg.Hq, cfg.Nq, cfg.D, dtype=dt, pin_memory=pin_memory)
    k = torch.empty(cfg.B, cfg.Hkv, cfg.N, cfg.D, dtype=dt, pin_memory=pin_memory)
    v = torch.empty(cfg.B, cfg.Hkv, cfg.N, cfg.D, dtype=dt, pin_memory=pin_memory)
    _fill(q, cfg, T_Q, cfg.Nq, hm, workers)
    _fill(k, cfg, T_K, cfg.N, hm, workers)
    _fill(v, cfg, T_V, cfg.N, hm, workers)
    return {"q": q, "k": k, "v": v}


def make_grads(cfg: Config, workers: int = 8) -> Dict[str, torch.Tensor]:
    """Upstream gradients d_full, d_sparse [B,Hq,Nq,D] (CPU, config dtype)."""
    dt = torch_dtype(cfg)
    hm = default_head_map(cfg.Hq, cfg.Hkv)
    out = {}
    for name, tid in (("d_full", T_DFULL), ("d_sparse", T_DSPARSE)):
        t = torch.empty(cfg.B, cfg.Hq, cfg.Nq, cfg.D, dtype=dt)
        _fill(t, cfg, tid, cfg.Nq, hm, workers)
        out[name] = t
    return out


def make_head(cfg: Config, b: int, hq: int, head_map=None) -> Dict[str, torch.Tensor]:
    """The Q slice of q head `hq` and the K, V slices of its kv head, for
    batch b (identical to the matching slices of make_inputs)."""
    hm = head_map if head_map is not None else default_head_map(cfg.Hq, cfg.Hkv)
    dt = torch_dtype(cfg)
    g = hm[hq]
    return {
        "q": _slice(cfg, T_Q, b, hq, cfg.Nq, hm).to(dt),
        "k": _slice(cfg, T_K, b, g, cfg.N, hm).to(dt),
        "v": _slice(cfg, T_V, b, g, cfg.N, hm).to(dt),
    }


def scale_for(cfg: Config) -> float:
    return 1.0 / math.sqrt(cfg.D)
