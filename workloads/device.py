"""Seeded input generators on the GPU (torch), for workloads too large to draw
on the host (multi-GB KV caches, 1 GB logits). Same distributions and storage
formats as ``workloads.gen``; tensors come from ``torch.Generator`` streams
seeded by (seed, stream id), so they are reproducible on one software stack
but not bit-equal to the NumPy host generators. Parity checks copy the slabs
they need back to the host.
"""

from __future__ import annotations

import torch

__all__ = ["dev_generator", "dev_kv_cache", "dev_queries", "dev_planted_logits", "dev_quantize_int8"]


def dev_generator(seed: int, stream: int, device="cuda") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed((int(seed) * 1_000_003 + int(stream)) & 0x7FFFFFFFFFFFFFFF)
    return g


def dev_quantize_int8(x: torch.Tensor):
    """Per-token symmetric int8 (last axis): scale = fp16(max|x| / 127),
    code = clip(round_half_even(x / scale), -127, 127); zero scale -> zero codes."""
    amax = x.abs().amax(dim=-1)
    scale = (amax / 127.0).to(torch.float16)
    s32 = scale.float().unsqueeze(-1)
    safe = torch.where(s32 > 0, s32, torch.ones_like(s32))
    q = torch.where(s32 > 0, torch.round(x / safe), torch.zeros_like(x))
    return q.clamp_(-127, 127).to(torch.int8), scale


def dev_kv_cache(seed: int, stream: int, B: int, Hkv: int, cap: int, D: int, dtype: str, device="cuda"):
    """One layer's K and V [B, Hkv, cap, D] ~ N(0, 1) in 'bf16' or 'i8' (+ fp16
    scales [B, Hkv, cap]); drawn one sequence at a time to bound temporaries."""
    out = {}
    for name, sid in (("k", 0), ("v", 1)):
        g = dev_generator(seed, stream * 16 + sid, device)
        if dtype == "bf16":
            t = torch.empty(B, Hkv, cap, D, dtype=torch.bfloat16, device=device)
            for b in range(B):
                t[b] = torch.randn(Hkv, cap, D, generator=g, device=device).to(torch.bfloat16)
            out[name] = t
        elif dtype == "i8":
            t = torch.empty(B, Hkv, cap, D, dtype=torch.int8, device=device)
            s = torch.empty(B, Hkv, cap, dtype=torch.float16, device=device)
            for b in range(B):
                code, scale = dev_quantize_int8(torch.randn(Hkv, cap, D, generator=g, device=device))
                t[b] = code
                s[b] = scale
            out[name] = t
            out[name + "_scale"] = s
        elif dtype == "f32":
            out[name] = torch.randn(B, Hkv, cap, D, generator=g, device=device)
        else:
            raise ValueError(dtype)
    return out


def dev_queries(seed: int, stream: int, n_nodes: int, Hq: int, D: int, dtype: str, device="cuda"):
    g = dev_generator(seed, 10_000 + stream, device)
    q = torch.randn(n_nodes, Hq, D, generator=g, device=device)
    return q if dtype == "f32" else q.to(torch.bfloat16)


def dev_planted_logits(seed: int, targets, vocab: int, sigma: float, device="cuda"):
    """fp32 [N, vocab] ~ N(0, sigma^2) with each row's unique maximum placed at
    targets[n] (set to the row's largest draw plus 1)."""
    g = dev_generator(seed, 20_000, device)
    t = torch.as_tensor(targets, dtype=torch.int64, device=device)
    x = torch.randn(len(t), vocab, generator=g, device=device).mul_(sigma)
    rows = torch.arange(len(t), device=device)
    x[rows, t] = x.amax(dim=1) + 1.0
    return x
