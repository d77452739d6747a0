"""Benchmark: one verify round = ancestor mask -> L x tree attention -> vocab
argmax -> accept walk -> in-place rollback gather, on synthetic inputs resident
in HBM. Prints one JSON line.

Default workload: the long-context stress round (B=8 sequences, 8 layers,
131,072-token prefix, 16-node confidence trees with worst-case scattered
accepted paths, int8 KV + fp16 per-token scales, 40/8 heads, head_dim 128,
vocab 248,320). --config 4 runs the batched ragged round instead (B=32, bf16,
prefixes U{1024..32768}, 8-64-node trees).
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=5, choices=[4, 5])
    ap.add_argument("--take-reps", type=int, default=3, help="timed reps of the full-window out-of-place gather")
    ap.add_argument("--no-take", action="store_true")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-heads", type=int, default=2, help="KV heads in the CPU oracle sample")
    return ap.parse_args()


def build_workload(cfg: int, dev: str):
    import numpy as np
    import torch

    import token_tree_verification_build_amd as ttv
    from workloads import config4_round, config5_round
    from workloads.device import dev_kv_cache, dev_planted_logits, dev_queries

    if cfg == 5:
        spec = config5_round(0, [131072] * 8, "tree")
    else:
        spec = config4_round()
    cap = int(max(spec.hist_len + np.diff(spec.node_off)))
    L = spec.L
    caches, layers, qs = [], [], []
    for l in range(L):
        c = dev_kv_cache(spec.seed, 100 + l, spec.B, spec.Hkv, cap, spec.D, spec.kv_dtype, dev)
        caches.append(c)
        layers.append(ttv.KVLayer(c["k"], c["v"], c.get("k_scale"), c.get("v_scale")))
        qs.append(dev_queries(spec.seed, 200 + l, spec.n_nodes, spec.Hq, spec.D, spec.q_dtype, dev))
    logits = dev_planted_logits(spec.seed, spec.flat_targets, spec.vocab, spec.sigma, dev)
    torch.cuda.synchronize()
    return spec, cap, caches, layers, qs, logits


def kv_row_bytes(spec) -> int:
    esz = {"f32": 4, "bf16": 2, "i8": 1}[spec.kv_dtype]
    return 2 * spec.D * esz + (4 if spec.kv_dtype == "i8" else 0)


def attention_bytes(spec) -> int:
    """Algorithmic HBM bytes of one attention launch: every K/V row (and int8
    scale) each sequence's unit reads once, plus Q in and O out."""
    import numpy as np
    rows = int(np.sum(spec.hist_len + np.diff(spec.node_off)))
    qbytes = spec.n_nodes * spec.Hq * spec.D * (2 if spec.q_dtype == "bf16" else 4)
    obytes = spec.n_nodes * spec.Hq * spec.D * 4
    return rows * spec.Hkv * kv_row_bytes(spec) + qbytes + obytes


def attention_flops(spec) -> int:
    import numpy as np
    total = 0
    for P, par in zip(spec.hist_len, spec.parents):
        depth = np.zeros(len(par), np.int64)
        for i in range(1, len(par)):
            depth[i] = depth[par[i]] + 1
        total += int(np.sum(int(P) + depth + 1))
    return 4 * spec.D * spec.Hq * total


def cpu_baseline(spec, caches, qs, logits, heads: int):
    """The oracle, untuned, on a bounded sample of the same round: layer 0,
    sequence 0, KV heads [0, heads), that sequence's argmax, walk and a
    one-layer rollback gather over the same heads; scaled to a full round."""
    import numpy as np

    import oracle as O

    b = 0
    P = int(spec.hist_len[b])
    o0, o1 = int(spec.node_off[b]), int(spec.node_off[b + 1])
    T = o1 - o0
    G = spec.G
    c = caches[0]
    lay = {}
    for n, t in c.items():
        sl = t[b:b + 1, :heads, :P + T]
        lay[n] = sl.view(torch_int16()).cpu().numpy().view(np.uint16) if str(t.dtype) == "torch.bfloat16" \
            else sl.cpu().numpy()
    q = qs[0][o0:o1, :heads * G]
    qh = q.view(torch_int16()).cpu().numpy().view(np.uint16) if spec.q_dtype == "bf16" else q.cpu().numpy()
    lg = logits[o0:o1].cpu().numpy()
    threads = len(os.sched_getaffinity(0))
    t0 = time.perf_counter()
    O.tree_verify_attention(qh, lay, np.array([0, T]), np.array([P]), [spec.parents[b]], 1 / math.sqrt(spec.D),
                            spec.q_dtype, spec.kv_dtype)
    t_attn = time.perf_counter() - t0
    t0 = time.perf_counter()
    am = O.vocab_argmax(lg)
    path, _ = O.tree_accept_walk(spec.parents[b], spec.tokens[b], am)
    t_walk = time.perf_counter() - t0
    t0 = time.perf_counter()
    O.gather_layer(lay, [O.rollback_selection(P, path)])
    t_gather = time.perf_counter() - t0
    scale = spec.Hkv / heads
    per_seq = spec.L * scale * (t_attn + t_gather) + t_walk
    round_s = per_seq * spec.B
    nodes = spec.n_nodes
    return {
        "value": nodes / round_s,
        "unit": "nodes/s",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"float64 NumPy oracle on layer 0, sequence 0, KV heads 0..{heads - 1} ({heads * G} query heads, "
                   f"{T} nodes, prefix {P}), plus that sequence's argmax/walk and a one-layer rollback gather of "
                   f"the same heads; {t_attn + t_walk + t_gather:.1f} s measured, scaled x{spec.L * scale * spec.B:.0f}"
                   f" to the full round"),
        "sample_seconds": round(t_attn + t_walk + t_gather, 2),
    }


def torch_int16():
    import torch
    return torch.int16


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        if int(os.environ.get("RANK", "0")) == 0:
            print("bench.py measures one GPU: the verify path runs on a single MI355X in this build; "
                  "--gpus must be 1 (how the path would shard is described in DESIGN.md)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import token_tree_verification_build_amd as ttv
    from workloads import CONFIG_TEXT

    dev = "cuda:0"
    torch.cuda.set_device(0)
    print(f"[bench] building config {args.config} workload", file=sys.stderr, flush=True)
    spec, cap, caches, layers, qs, logits = build_workload(args.config, dev)
    B, L, n = spec.B, spec.L, spec.n_nodes
    batch = ttv.Batch(spec.node_off, spec.hist_len, device=dev)
    parent = torch.from_numpy(spec.flat("parents")).to(dev)
    token = torch.from_numpy(spec.flat("tokens").astype(np.int32)).to(dev)
    st = torch.zeros(1, dtype=torch.int32, device=dev)
    anc = torch.empty(n, dtype=torch.int64, device=dev)
    depth = torch.empty(n, dtype=torch.int32, device=dev)
    out = torch.empty(n, spec.Hq, spec.D, dtype=torch.float32, device=dev)
    ws = torch.zeros(ttv.tree_verify_attention_ws(batch, spec.Hq, layers[0], spec.q_dtype), dtype=torch.uint8,
                     device=dev)
    am = torch.empty(n, dtype=torch.int32, device=dev)
    aws = torch.zeros(max(1, ttv.vocab_argmax_ws(n, spec.vocab)), dtype=torch.uint8, device=dev)
    path = torch.empty(B, 64, dtype=torch.int32, device=dev)
    plen = torch.empty(B, dtype=torch.int32, device=dev)
    emitted = torch.empty(B, 64, dtype=torch.int32, device=dev)
    sel = torch.empty(B, cap, dtype=torch.int32, device=dev)
    sel_len = torch.empty(B, dtype=torch.int32, device=dev)
    live = (spec.hist_len + np.diff(spec.node_off)).astype(np.int32)
    gws = torch.zeros(ttv.kv_gather_positions_ws(B), dtype=torch.uint8, device=dev)
    scale = 1.0 / math.sqrt(spec.D)

    def step():
        ttv.tree_build_mask(batch, parent, anc, depth, st)
        for l in range(L):
            ttv.tree_verify_attention(batch, qs[l], layers[l], anc, scale, out, ws)
        ttv.vocab_argmax(logits, am, aws)
        ttv.tree_accept_walk(batch, parent, token, am, path, plen, emitted, st, sel, sel_len)
        ttv.kv_gather_positions(layers, None, sel, sel_len, live, st, gws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    assert int(st.item()) == 0, "device status after warmup"
    print(f"[bench] warmup done; timing {args.steps} steps", file=sys.stderr, flush=True)

    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record()
    for _ in range(args.steps):
        step()
    t_end.record()
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    ms_per_step = total_ms / args.steps
    nodes_per_s = n * args.steps / (total_ms / 1e3)

    # attention launches: average duration over steps x layers, timed with events on the launch stream
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps * L)]
    torch.cuda.synchronize()
    for s in range(args.steps):
        for l in range(L):
            e0, e1 = evs[s * L + l]
            e0.record()
            ttv.tree_verify_attention(batch, qs[l], layers[l], anc, scale, out, ws)
            e1.record()
    torch.cuda.synchronize()
    attn_ms = sum(e0.elapsed_time(e1) for e0, e1 in evs) / len(evs)
    abytes = attention_bytes(spec)
    aflops = attention_flops(spec)
    attn_gbs = abytes / (attn_ms / 1e3) / 1e9
    print(f"[bench] step {ms_per_step:.3f} ms; attention {attn_ms * 1e3:.1f} us/launch "
          f"({attn_gbs:.0f} GB/s, {aflops / (attn_ms / 1e3) / 1e12:.0f} TFLOP/s)", file=sys.stderr, flush=True)

    kernels = {
        "tree_verify_attention": {
            "avg_us": round(attn_ms * 1e3, 2), "bytes": abytes, "GBps": round(attn_gbs, 1),
            "frac_hbm": round(attn_gbs / HBM_PEAK_GBS, 4), "flops": aflops,
            "TFLOPs": round(aflops / (attn_ms / 1e3) / 1e12, 1),
        }
    }

    # full-window out-of-place gather (the pages' take): every survivor of every layer rewritten
    if not args.no_take:
        dst_caches = [{k: torch.empty_like(t) for k, t in c.items()} for c in caches]
        dst_layers = [ttv.KVLayer(c["k"], c["v"], c.get("k_scale"), c.get("v_scale")) for c in dst_caches]
        torch.cuda.synchronize()
        ttv.kv_gather_positions(layers, dst_layers, sel, sel_len, live, st, gws)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(args.take_reps):
            ttv.kv_gather_positions(layers, dst_layers, sel, sel_len, live, st, gws)
        e1.record()
        torch.cuda.synchronize()
        take_ms = e0.elapsed_time(e1) / args.take_reps
        rows = int(sel_len.sum().item())
        tbytes = 2 * rows * spec.Hkv * kv_row_bytes(spec) * L + rows * 4 * 2
        kernels["kv_gather_positions_take"] = {
            "avg_us": round(take_ms * 1e3, 1), "bytes": tbytes, "GBps": round(tbytes / (take_ms / 1e3) / 1e9, 1),
            "frac_hbm": round(tbytes / (take_ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
            "what": "out-of-place full-window take of all layers (validate + copy launches)",
        }
        print(f"[bench] full-window take {take_ms:.3f} ms ({kernels['kv_gather_positions_take']['GBps']} GB/s)",
              file=sys.stderr, flush=True)
        del dst_caches, dst_layers
    assert int(st.item()) == 0, "device status"

    cpu = None
    if not args.no_cpu:
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        cpu = cpu_baseline(spec, caches, qs, logits, args.cpu_heads)

    res = {
        "metric": "verified tree nodes/sec + achieved HBM GB/s (verify attn, KV gather) on 1 MI355X",
        "value": round(nodes_per_s, 1),
        "unit": "nodes/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "kv_storage": "int8 + fp16 per-token scales" if spec.kv_dtype == "i8" else spec.kv_dtype,
        "data": "synthetic",
        "config": {"workload": CONFIG_TEXT[args.config], "batch": B, "layers": L,
                   "prefix": [int(spec.hist_len.min()), int(spec.hist_len.max())], "nodes_per_round": n,
                   "Hq": spec.Hq, "Hkv": spec.Hkv, "head_dim": spec.D, "vocab": spec.vocab,
                   "step": "mask + L x attention + argmax + walk + in-place rollback gather"},
        "roofline": {"bound": "hbm", "achieved": round(attn_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(attn_gbs / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "tree_verify_attention"},
        "cpu_baseline": cpu,
        "kernels": kernels,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
