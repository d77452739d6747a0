"""Helpers for the GPU parity tests: upload seeded host inputs, run the
library's steps through the Python binding, bring results back."""

from __future__ import annotations

import sys

import numpy as np
import torch

DEV = "cuda"


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def binding():
    import token_tree_verification_build_amd as ttv  # raises if libttv.so is missing
    return ttv


def to_dev(a, kind: str | None = None):
    """numpy -> device tensor; kind 'bf16' reinterprets uint16 bit patterns."""
    a = np.ascontiguousarray(a)
    if kind == "bf16" or (kind is None and a.dtype == np.uint16):
        return torch.from_numpy(a.view(np.int16)).to(DEV).view(torch.bfloat16)
    if a.dtype == np.uint64:
        return torch.from_numpy(a.view(np.int64)).to(DEV)
    return torch.from_numpy(a).to(DEV)


def to_host(t):
    """device tensor -> numpy (bf16 as uint16 bits, int64 anc as uint64)."""
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def layer_to_dev(ttv, host_layer: dict):
    d = {}
    for name, arr in host_layer.items():
        if name == "q":
            continue
        d[name] = to_dev(arr)
    return d, ttv.KVLayer(d["k"], d["v"], d.get("k_scale"), d.get("v_scale"))


def layer_to_host(dev_layer: dict) -> dict:
    return {n: to_host(t) for n, t in dev_layer.items()}


def zeros_ws(nbytes: int):
    return torch.zeros(max(int(nbytes), 1), dtype=torch.uint8, device=DEV)


def status():
    return torch.zeros(1, dtype=torch.int32, device=DEV)


def run_attention(ttv, batch, q_dev, kv_layer, anc_dev, scale: float, ws=None):
    n, Hq, D = q_dev.shape
    qd = "f32" if q_dev.dtype == torch.float32 else "bf16"
    need = ttv.tree_verify_attention_ws(batch, Hq, kv_layer, qd)
    assert need > 0, ttv.last_error()
    if ws is None or ws.numel() < need:
        ws = zeros_ws(need)
    out = torch.full((n, Hq, D), float("nan"), dtype=torch.float32, device=DEV)
    ttv.tree_verify_attention(batch, q_dev, kv_layer, anc_dev, scale, out, ws)
    return out, ws


def run_argmax(ttv, logits_dev):
    n, V = logits_dev.shape
    ws = zeros_ws(ttv.vocab_argmax_ws(n, V))
    out = torch.full((n,), -7, dtype=torch.int32, device=DEV)
    ttv.vocab_argmax(logits_dev, out, ws)
    return out


def run_mask(ttv, batch, parent_dev):
    n = parent_dev.numel()
    anc = torch.full((max(n, 1),), -1, dtype=torch.int64, device=DEV)
    depth = torch.full((max(n, 1),), -5, dtype=torch.int32, device=DEV)
    st = status()
    ttv.tree_build_mask(batch, parent_dev, anc, depth, st)
    return anc, depth, st


def run_walk(ttv, batch, parent_dev, token_dev, argmax_dev, with_sel=True):
    B = batch.B
    path = torch.full((B, 64), -3, dtype=torch.int32, device=DEV)
    plen = torch.full((B,), -3, dtype=torch.int32, device=DEV)
    emitted = torch.full((B, 64), -3, dtype=torch.int32, device=DEV)
    st = status()
    sel = sel_len = None
    if with_sel:
        stride = int(max(batch.hist_len_h + np.diff(batch.node_off_h))) if B else 1
        sel = torch.full((B, stride), -9, dtype=torch.int32, device=DEV)
        sel_len = torch.full((B,), -9, dtype=torch.int32, device=DEV)
    ttv.tree_accept_walk(batch, parent_dev, token_dev, argmax_dev, path, plen, emitted, st, sel, sel_len)
    return path, plen, emitted, sel, sel_len, st


def spec_batch(ttv, spec):
    return ttv.Batch(spec.node_off, spec.hist_len)
