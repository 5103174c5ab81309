"""Seeded synthetic inputs with the attention shapes of the measured workloads.

Shared by the tests, the benchmark and the smoke check; it computes nothing of
the method itself (no summaries, scores, selection or attention), only draws
random tensors and lays them out.  Every stream of randomness (keys, values,
queries, heavy-block choice, query drift) has its own torch generator seeded
from the workload's base seed, so each tensor is reproducible on its own.

Stand-ins: the pages' accuracy and serving runs use real Qwen3 / Llama-3.1
models with EAGLE-3 draft heads on GSM8K, AIME, GPQA-Diamond and LongBench v2.
None of that is used; only the attention shapes are kept, with
  keys, values, queries ~ N(0, 1);
  heavy blocks: round(0.05 * n) distinct blocks per (request, KV head) whose
    keys are shifted by +2 along the unit vector of the mean of that KV head's
    normal query heads (so a few blocks carry most of the attention mass);
  draft query = 0.98 * q + 0.2 * N(0, 1);
  drift between decode steps: q' = rho * q + sqrt(1 - rho^2) * N(0, 1).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    R: int          # requests (batch)
    Hq: int         # query heads
    H: int          # KV heads
    D: int          # head dim
    L: int          # context tokens per request
    B: int          # block size
    K: int          # top-K blocks = resident slots per KV head
    dtype: torch.dtype
    heavy: bool     # heavy-block key structure
    seed: int
    n_q: int = 2    # stacked rows: normal + draft
    layers: int = 1
    steps: int = 0
    cap: int = 16
    rho: float = 0.98

    @property
    def G(self) -> int:
        return self.Hq // self.H

    @property
    def n_blk(self) -> int:
        return self.L // self.B


WORKLOADS = {
    "tiny-fp32": Workload("tiny-fp32", R=1, Hq=2, H=1, D=64, L=1024, B=16, K=8,
                          dtype=torch.float32, heavy=False, seed=20260001),
    "qwen3-8b-1layer": Workload("qwen3-8b-1layer", R=1, Hq=32, H=8, D=128, L=32768, B=16,
                                K=128, dtype=torch.bfloat16, heavy=True, seed=20260002),
    "llama3.1-8b-32layer": Workload("llama3.1-8b-32layer", R=32, Hq=32, H=8, D=128, L=32768,
                                    B=16, K=128, dtype=torch.bfloat16, heavy=True,
                                    seed=20260003, layers=32, steps=100, cap=16),
    "qwen3-235b-1layer": Workload("qwen3-235b-1layer", R=8, Hq=64, H=4, D=128, L=131072, B=16,
                                  K=128, dtype=torch.bfloat16, heavy=True, seed=20260004),
    "qwen3-8b-pipeline": Workload("qwen3-8b-pipeline", R=8, Hq=32, H=8, D=128, L=32768, B=16,
                                  K=128, dtype=torch.bfloat16, heavy=True, seed=20260005,
                                  layers=36, steps=200, cap=16),
}

# Independent random streams of one workload.
S_KEYS, S_VALUES, S_QUERY, S_HEAVY, S_DRIFT, S_MISC = range(6)


def workload(name: str, **overrides) -> Workload:
    return replace(WORKLOADS[name], **overrides)


def generator(seed: int, stream: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) * 64 + int(stream))
    return g


def normal(shape, gen: torch.Generator, device, dtype=torch.float32) -> torch.Tensor:
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float32).to(dtype)


def queries(wl: Workload, device, layer: int = 0, gen: torch.Generator | None = None):
    """Stacked [normal; draft] queries [R][2][Hq][D] in fp32 (cast by the caller)."""
    g = gen or generator(wl.seed + 1000 * layer, S_QUERY, device)
    q = torch.randn((wl.R, wl.Hq, wl.D), generator=g, device=device)
    d = 0.98 * q + 0.2 * torch.randn((wl.R, wl.Hq, wl.D), generator=g, device=device)
    return torch.stack([q, d], dim=1)


def drift(q_normal: torch.Tensor, rho: float, gen: torch.Generator):
    """Next step's stacked queries from this step's normal query [R][Hq][D] (fp32)."""
    eps = torch.randn(q_normal.shape, generator=gen, device=q_normal.device)
    qn = rho * q_normal + math.sqrt(1.0 - rho * rho) * eps
    dr = 0.98 * qn + 0.2 * torch.randn(q_normal.shape, generator=gen, device=q_normal.device)
    return torch.stack([qn, dr], dim=1)


def keys(wl: Workload, q_normal: torch.Tensor | None, device, layer: int = 0,
         out: torch.Tensor | None = None) -> torch.Tensor:
    """Keys [R][H][L][D] in wl.dtype.  With wl.heavy, q_normal [R][Hq][D] fixes the
    shift direction of each KV head's heavy blocks."""
    g = generator(wl.seed + 1000 * layer, S_KEYS, device)
    gh = generator(wl.seed + 1000 * layer, S_HEAVY, device)
    if out is None:
        out = torch.empty((wl.R, wl.H, wl.L, wl.D), dtype=wl.dtype, device=device)
    n_heavy = int(round(0.05 * wl.n_blk))
    for r in range(wl.R):
        k = torch.randn((wl.H, wl.L, wl.D), generator=g, device=device)
        if wl.heavy and n_heavy > 0:
            qg = q_normal[r].float().view(wl.H, wl.G, wl.D).mean(dim=1)
            u = qg / qg.norm(dim=-1, keepdim=True).clamp_min(1e-30)
            kb = k.view(wl.H, wl.n_blk, wl.B, wl.D)
            for h in range(wl.H):
                pick = torch.randperm(wl.n_blk, generator=gh, device=device)[:n_heavy]
                kb[h, pick] += 2.0 * u[h]
        out[r].copy_(k.to(wl.dtype))
    return out


def values(wl: Workload, device, layer: int = 0, out: torch.Tensor | None = None) -> torch.Tensor:
    """Values [R][H][L][D] in wl.dtype (token-major; see v_tiles for the stored layout)."""
    g = generator(wl.seed + 1000 * layer, S_VALUES, device)
    if out is None:
        out = torch.empty((wl.R, wl.H, wl.L, wl.D), dtype=wl.dtype, device=device)
    for r in range(wl.R):
        out[r].copy_(torch.randn((wl.H, wl.L, wl.D), generator=g, device=device).to(wl.dtype))
    return out


def v_tiles(v: torch.Tensor, block_size: int) -> torch.Tensor:
    """Token-major values [..][L][D] -> dim-major V tiles [..][L/B][D][B]."""
    *lead, L, D = v.shape
    B = int(block_size)
    return v.reshape(*lead, L // B, B, D).transpose(-1, -2).contiguous()


def v_tiles_to_tokens(vt: torch.Tensor) -> torch.Tensor:
    """Dim-major V tiles [..][n][D][B] -> token-major values [..][n*B][D]."""
    *lead, n, D, B = vt.shape
    return vt.transpose(-1, -2).reshape(*lead, n * B, D)


def interleave_kv(kt: torch.Tensor, vt: torch.Tensor, out: torch.Tensor | None = None):
    """Pack K tiles [..][n][B][D] and dim-major V tiles [..][n][D][B] into one
    interleaved store [..][n][2][B][D] (each block-head's K tile, then its V
    tile).  Returns (store, K view, V view); the views are what the kernels take."""
    *lead, B, D = kt.shape
    if out is None:
        out = torch.empty((*lead, 2, B, D), dtype=kt.dtype, device=kt.device)
    out[..., 0, :, :] = kt
    out[..., 1, :, :] = vt.reshape(*lead, B, D)  # same bytes, V tile order kept
    flat = out.view(*lead, 2, B * D)
    return out, out[..., 0, :, :], flat[..., 1, :].unflatten(-1, (D, B))


def random_tile_table(R: int, H: int, n_sel: int, n_blk: int, gen: torch.Generator,
                      device) -> torch.Tensor:
    """Distinct block ids per (request, KV head): [R][H][n_sel] int32."""
    t = torch.empty((R, H, n_sel), dtype=torch.int32, device=device)
    for r in range(R):
        for h in range(H):
            t[r, h] = torch.randperm(n_blk, generator=gen, device=device)[:n_sel].to(torch.int32)
    return t
