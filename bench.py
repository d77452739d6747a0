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
    ap.add_argument("--no-small", action="store_true", help="skip the tiny, chain and 16-layer int8 round timings")
    ap.add_argument("--no-window", action="store_true",
                    help="skip the sliding-window layer timing (its launches share the attention kernels' names, so "
                         "counter and trace summaries of the full-context call leave it out)")
    ap.add_argument("--cpu-heads", type=int, default=8, help="KV heads per sampled sequence in the CPU oracle sample")
    ap.add_argument("--cpu-seqs", type=int, default=2, help="sequences in the CPU oracle sample")
    ap.add_argument("--copy-calib-mib", type=int, default=0,
                    help="after the timed region, run one plain device copy of this many MiB (the reference "
                         "dispatch that scales FETCH_SIZE / WRITE_SIZE counters to bytes)")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="summarise two rocprofv3 --pmc counter CSVs (FETCH_SIZE run, WRITE_SIZE run) of "
                         "'bench.py --copy-calib-mib N' into HBM traffic per kernel, then exit")
    ap.add_argument("--calib-mib", type=int, default=1024, help="the --copy-calib-mib of the summarised runs")
    ap.add_argument("--sq-summary", metavar="SQ_CSV",
                    help="summarise a rocprofv3 --pmc counter CSV of SQ_VALU_MFMA_BUSY_CYCLES, SQ_ACTIVE_INST_VALU, "
                         "SQ_VALU_MFMA_COEXEC_CYCLES, SQ_BUSY_CYCLES, SQ_WAIT_INST_ANY, SQ_ACTIVE_INST_LDS, "
                         "SQ_INSTS_VALU, SQ_INSTS_MFMA and GRBM_GUI_ACTIVE into per-kernel MFMA / VALU busy "
                         "fractions, then exit")
    ap.add_argument("--trace-summary", metavar="KERNEL_STATS_CSV",
                    help="print the library's kernels from a rocprofv3 --kernel-trace --stats kernel_stats.csv "
                         "(durations in microseconds), then exit")
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


def cpu_baseline(spec, caches, qs, logits, heads: int, seqs: int):
    """The oracle, untuned, on a bounded sample of the same round: layer 0,
    sequences [0, seqs), KV heads [0, heads) of each, each sequence's argmax,
    walk and a one-layer rollback gather over the same heads; scaled to a
    full round."""
    import numpy as np

    import oracle as O

    G = spec.G
    c = caches[0]
    threads = len(os.sched_getaffinity(0))
    t_attn = t_walk = t_gather = 0.0
    for b in range(seqs):
        P = int(spec.hist_len[b])
        o0, o1 = int(spec.node_off[b]), int(spec.node_off[b + 1])
        T = o1 - o0
        lay = {}
        for n, t in c.items():
            sl = t[b:b + 1, :heads, :P + T]
            lay[n] = sl.view(torch_int16()).cpu().numpy().view(np.uint16) if str(t.dtype) == "torch.bfloat16" \
                else sl.cpu().numpy()
        q = qs[0][o0:o1, :heads * G]
        qh = q.view(torch_int16()).cpu().numpy().view(np.uint16) if spec.q_dtype == "bf16" else q.cpu().numpy()
        lg = logits[o0:o1].cpu().numpy()
        t0 = time.perf_counter()
        O.tree_verify_attention(qh, lay, np.array([0, T]), np.array([P]), [spec.parents[b]], 1 / math.sqrt(spec.D),
                                spec.q_dtype, spec.kv_dtype)
        t_attn += time.perf_counter() - t0
        t0 = time.perf_counter()
        am = O.vocab_argmax(lg)
        path, _ = O.tree_accept_walk(spec.parents[b], spec.tokens[b], am)
        t_walk += time.perf_counter() - t0
        t0 = time.perf_counter()
        O.gather_layer(lay, [O.rollback_selection(P, path)])
        t_gather += time.perf_counter() - t0
        del lay
    scale = spec.Hkv / heads
    sampled = t_attn + t_walk + t_gather
    round_s = (spec.L * scale * (t_attn + t_gather) + t_walk) * spec.B / seqs
    nodes = spec.n_nodes
    return {
        "value": nodes / round_s,
        "unit": "nodes/s",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"float64 NumPy oracle on layer 0 of sequences 0..{seqs - 1}, KV heads 0..{heads - 1} of each "
                   f"({heads * G} query heads, prefix {int(spec.hist_len[:seqs].min())}..{int(spec.hist_len[:seqs].max())}), "
                   f"plus each sequence's argmax/walk and a one-layer rollback gather of the same heads; "
                   f"{sampled:.1f} s measured, attention and gather scaled x{spec.L * scale * spec.B / seqs:.0f} "
                   f"and argmax/walk x{spec.B / seqs:.0f} to the full round"),
        "sample_seconds": round(sampled, 2),
    }


def small_rounds(dev: str, steps: int = 100) -> dict:
    """One verify round per step for the tiny fp32 workload, the linear chains
    (T = 3, 4, 8) and the 16-node int8 tree over 16 layers, each timed with
    events over `steps` rounds. The chain and int8-tree workloads fit in the
    256 MB Infinity Cache, so every step takes the next of a rotation of
    buffer copies that together hold at least 1 GiB; the tiny round is
    latency-bound and reported as it is. Also the attention-only cost of a
    chain of T = 4 and T = 8 nodes relative to T = 1 at the chain shape."""
    import numpy as np
    import torch

    import token_tree_verification_build_amd as ttv
    from workloads import config1_round, config2_round, config3_round, host_tensors
    from workloads.device import dev_kv_cache, dev_planted_logits, dev_queries

    def timed(fn, n):
        for i in range(3):
            fn(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(n):
            fn(i)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n * 1e3  # us

    def graph_timed(fn, ncopies, n):
        """The same steps captured once per rotation copy as HIP graphs
        (torch.cuda.CUDAGraph over the library's launches), replayed in turn:
        the per-step launch cost without the host's per-launch overhead."""
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        graphs = []
        for i in range(ncopies):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=side):
                fn(i)
            graphs.append(g)
        torch.cuda.current_stream().wait_stream(side)
        for g in graphs:
            g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(n):
            graphs[i % ncopies].replay()
        e1.record()
        torch.cuda.synchronize()
        del graphs
        return e0.elapsed_time(e1) / n * 1e3  # us

    def round_runner(spec, layer_sets, q_sets, logit_sets):
        """step(i): mask + attention per layer + argmax + walk + in-place
        gather on rotation copy i % len(layer_sets)."""
        B = spec.B
        batch = ttv.Batch(spec.node_off, spec.hist_len, device=dev)
        parent = torch.from_numpy(spec.flat("parents")).to(dev)
        token = torch.from_numpy(spec.flat("tokens").astype(np.int32)).to(dev)
        n = spec.n_nodes
        st = torch.zeros(1, dtype=torch.int32, device=dev)
        anc = torch.empty(n, dtype=torch.int64, device=dev)
        out = torch.empty(n, spec.Hq, spec.D, dtype=torch.float32, device=dev)
        ws = torch.zeros(ttv.tree_verify_attention_ws(batch, spec.Hq, layer_sets[0][0], spec.q_dtype),
                         dtype=torch.uint8, device=dev)
        am = torch.empty(n, dtype=torch.int32, device=dev)
        aws = torch.zeros(max(1, ttv.vocab_argmax_ws(n, spec.vocab)), dtype=torch.uint8, device=dev)
        path = torch.empty(B, 64, dtype=torch.int32, device=dev)
        plen = torch.empty(B, dtype=torch.int32, device=dev)
        emitted = torch.empty(B, 64, dtype=torch.int32, device=dev)
        cap = int(max(spec.hist_len + np.diff(spec.node_off)))
        sel = torch.empty(B, cap, dtype=torch.int32, device=dev)
        sel_len = torch.empty(B, dtype=torch.int32, device=dev)
        live = (spec.hist_len + np.diff(spec.node_off)).astype(np.int32)
        gws = torch.zeros(ttv.kv_gather_positions_ws(B), dtype=torch.uint8, device=dev)
        scale = 1.0 / math.sqrt(spec.D)

        def step(i):
            layers, qs, logits = layer_sets[i % len(layer_sets)], q_sets[i % len(q_sets)], logit_sets[i % len(logit_sets)]
            ttv.tree_build_mask(batch, parent, anc, None, st)
            for l, lay in enumerate(layers):
                ttv.tree_verify_attention(batch, qs[l], lay, anc, scale, out, ws)
            ttv.vocab_argmax(logits, am, aws)
            ttv.tree_accept_walk(batch, parent, token, am, path, plen, emitted, st, sel, sel_len)
            ttv.kv_gather_positions(layers, None, sel, sel_len, live, st, gws)
        return step

    def rotation(nbytes_per_copy):
        return max(1, -(-(1 << 30) // max(1, nbytes_per_copy)))

    res = {}
    # tiny fp32 round (latency-bound; no rotation)
    spec = config1_round(accepted=2)
    tens = host_tensors(spec)
    L0 = tens["layers"][0]
    k = torch.from_numpy(L0["k"]).to(dev)
    v = torch.from_numpy(L0["v"]).to(dev)
    step = round_runner(spec, [[ttv.KVLayer(k, v)]], [[torch.from_numpy(L0["q"]).to(dev)]],
                        [torch.from_numpy(tens["logits"]).to(dev)])
    us = timed(step, steps)
    gus = graph_timed(step, 1, steps)
    res["config1"] = {"us_per_step": round(us, 2), "nodes_per_s": round(spec.n_nodes / us * 1e6, 1),
                      "us_per_step_graph": round(gus, 2), "nodes_per_s_graph": round(spec.n_nodes / gus * 1e6, 1),
                      "nodes": spec.n_nodes, "rotation_copies": 1,
                      "what": "7-node fp32 tree, 4/2 heads, D 64, prefix 64, vocab 1024"}
    # linear chains over a 2048-token bf16 prefix, and the chain-shape attention cost ratios
    attn_us = {}
    for T in (1, 3, 4, 8):
        spec = config2_round(T, T // 2)
        cap = int(spec.hist_len[0]) + T
        c = dev_kv_cache(spec.seed, 100, 1, spec.Hkv, cap, spec.D, "bf16", dev)
        per_copy = 2 * c["k"].numel() * 2 + T * spec.vocab * 4
        nrot = rotation(per_copy)
        kvs = [(c["k"].clone(), c["v"].clone()) for _ in range(nrot)]
        layer_sets = [[ttv.KVLayer(a, b)] for a, b in kvs]
        q = dev_queries(spec.seed, 200, T, spec.Hq, spec.D, "bf16", dev)
        logits = dev_planted_logits(spec.seed, spec.flat_targets, spec.vocab, spec.sigma, dev)
        logit_sets = [logits.clone() for _ in range(nrot)]
        if T > 1:
            step = round_runner(spec, layer_sets, [[q]], logit_sets)
            us = timed(step, max(steps, 2 * nrot))
            gus = graph_timed(step, nrot, max(steps, 2 * nrot))
            res[f"config2_T{T}"] = {"us_per_step": round(us, 2), "nodes_per_s": round(T / us * 1e6, 1), "nodes": T,
                                    "us_per_step_graph": round(gus, 2), "nodes_per_s_graph": round(T / gus * 1e6, 1),
                                    "rotation_copies": nrot, "rotated_bytes": nrot * per_copy,
                                    "what": f"chain of {T} nodes, bf16, 40/8 heads, prefix 2048, vocab 248320"}
        batch = ttv.Batch(spec.node_off, spec.hist_len, device=dev)
        out = torch.empty(T, spec.Hq, spec.D, dtype=torch.float32, device=dev)
        ws = torch.zeros(max(1, ttv.tree_verify_attention_ws(batch, spec.Hq, layer_sets[0][0], "bf16")),
                         dtype=torch.uint8, device=dev)
        attn_us[T] = timed(lambda i: ttv.tree_verify_attention(batch, q, layer_sets[i % nrot][0], None,
                                                               1 / math.sqrt(spec.D), out, ws), max(steps, 2 * nrot))
        del kvs, layer_sets, logit_sets
    res["verify_cost_ratio"] = {
        "attention_us": {f"T{T}": round(u, 2) for T, u in attn_us.items()},
        "T4_over_T1": round(attn_us[4] / attn_us[1], 3), "T8_over_T1": round(attn_us[8] / attn_us[1], 3),
        "context_pages": {"T4_over_T1": 1.29, "T8_over_T1": 2.48, "what": "whole verify forward, Apple M5 Max, "
                          "4-bit 27B target: context only, not a like-for-like comparison"},
        "what": "attention only (causal chain), bf16 KV, 40/8 heads, prefix 2048, rotated over >= 1 GiB"}
    # 16-node int8 tree over 16 layers
    spec = config3_round()
    cap = int(spec.hist_len[0]) + spec.n_nodes
    base = [dev_kv_cache(spec.seed, 100 + l, 1, spec.Hkv, cap, spec.D, "i8", dev) for l in range(spec.L)]
    per_copy = sum(t.numel() * t.element_size() for c in base for t in c.values()) + spec.n_nodes * spec.vocab * 4
    nrot = rotation(per_copy)
    copies = [[{n: t.clone() for n, t in c.items()} for c in base] for _ in range(nrot)]
    layer_sets = [[ttv.KVLayer(c["k"], c["v"], c["k_scale"], c["v_scale"]) for c in cp] for cp in copies]
    qs = [dev_queries(spec.seed, 200 + l, spec.n_nodes, spec.Hq, spec.D, "bf16", dev) for l in range(spec.L)]
    logits = dev_planted_logits(spec.seed, spec.flat_targets, spec.vocab, spec.sigma, dev)
    step = round_runner(spec, layer_sets, [qs], [logits.clone() for _ in range(nrot)])
    us = timed(step, max(steps, 2 * nrot))
    gus = graph_timed(step, nrot, max(steps, 2 * nrot))
    res["config3"] = {"us_per_step": round(us, 2), "nodes_per_s": round(spec.n_nodes / us * 1e6, 1),
                      "us_per_step_graph": round(gus, 2), "nodes_per_s_graph": round(spec.n_nodes / gus * 1e6, 1),
                      "nodes": spec.n_nodes, "rotation_copies": nrot, "rotated_bytes": nrot * per_copy,
                      "what": "16-node int8 tree, 16 layers, 40/8 heads, prefix 4096, vocab 248320"}
    del copies, layer_sets, base
    torch.cuda.empty_cache()
    return res


ATTN_SOURCE = os.path.join(ROOT, "token_tree_verification_build_amd", "csrc", "attention.hip")
# counter summaries per workload, named for the kernel and the workload they cover
PROFILE_STEM = {5: "tree_verify_attention_i8_131k", 4: "tree_verify_attention_bf16_ragged_b32"}
TRAFFIC_TAG = "bench-traffic: "
# the kernels one tree_verify_attention call launches (main kernels of every
# path, the exact int8 pass and the split-KV merge)
ATTN_KERNELS = ("attn_i8_split_kernel", "attn_bf16_split_kernel", "attn_bf16_narrow_kernel", "attn_valu_kernel",
                "merge_kernel")


def is_attention_kernel(name: str) -> bool:
    return any(k in name for k in ATTN_KERNELS)


def profile_file(config: int, what: str) -> str:
    return os.path.join(ROOT, "profiles", f"{PROFILE_STEM[config]}_{what}.txt")


def source_digest(path: str) -> str:
    """SHA-256 of the source's code: every line with its // comment and
    surrounding blanks removed, empty lines dropped (a comment edit leaves
    recorded counters valid; any code change invalidates them)."""
    import hashlib
    code = []
    with open(path, encoding="utf-8") as f:
        for line in f:
            out, in_str, i = [], False, 0
            while i < len(line):
                ch = line[i]
                if ch == '"' and (i == 0 or line[i - 1] != "\\"):
                    in_str = not in_str
                elif not in_str and line.startswith("//", i):
                    break
                out.append(ch)
                i += 1
            t = "".join(out).strip()
            if t:
                code.append(t)
    return hashlib.sha256("\n".join(code).encode()).hexdigest()


def pmc_rows(csv_path: str, counter: str) -> dict:
    """Kernel name -> list of per-dispatch counter values (KiB) from a rocprofv3 counter CSV."""
    import csv
    out: dict = {}
    with open(csv_path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] == counter:
                out.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return out


def pmc_summary(fetch_csv: str, write_csv: str, calib_mib: int) -> None:
    """HBM traffic per dispatch. FETCH_SIZE and WRITE_SIZE (KiB per dispatch) are
    each scaled by the bytes-per-KiB that the same counter reads for the plain
    copy of calib_mib MiB (which reads and writes exactly that many bytes)."""
    fetch, write = pmc_rows(fetch_csv, "FETCH_SIZE"), pmc_rows(write_csv, "WRITE_SIZE")
    nbytes = calib_mib << 20

    def copy_value(rows):
        # the calibration copy is a runtime buffer copy (torch's own copy
        # kernels, e.g. dtype conversions, are not calibrated transfers)
        cands = [(k, v) for k, v in rows.items() if "copybuffer" in k.lower()]
        cands = cands or [(k, v) for k, v in rows.items() if "copy" in k.lower()]
        # the calibration copy is the dispatch whose counter reads closest to its size
        k, v = min(cands, key=lambda kv: abs(max(kv[1]) * 1024 - nbytes))
        return k, max(v)

    ck, cf = copy_value(fetch)
    _, cw = copy_value(write)
    f_scale, w_scale = nbytes / (cf * 1024), nbytes / (cw * 1024)
    print(f"calibration copy: {ck[:100]}")
    print(f"  {calib_mib} MiB copied; FETCH_SIZE {cf:.0f} KiB -> {f_scale:.4f} B per counted B; "
          f"WRITE_SIZE {cw:.0f} KiB -> {w_scale:.4f} B per counted B")
    print(f"{'kernel':90s} {'n':>4s} {'fetch MB':>10s} {'write MB':>10s} {'scaled MB':>10s}")
    # the attention call = every kernel it launches, each dispatched once per
    # call (per-dispatch means add up to the call's bytes)
    main, top, rd, wr = None, -1.0, 0.0, 0.0
    for k in sorted(set(fetch) & set(write)):
        if "ttv::" not in k and k != ck:   # the library's kernels and the calibration copy
            continue
        fv, wv = fetch[k], write[k]
        fm, wm = sum(fv) / len(fv) * 1024, sum(wv) / len(wv) * 1024
        tot = fm * f_scale + wm * w_scale
        print(f"{k[:90]:90s} {len(fv):4d} {fm / 1e6:10.2f} {wm / 1e6:10.2f} {tot / 1e6:10.2f}")
        if is_attention_kernel(k):
            rd, wr = rd + fm * f_scale, wr + wm * w_scale
            if "merge_kernel" not in k and tot > top:
                main, top = k, tot
    if main is not None:
        rec = {"kernel": main, "traffic_bytes": round(rd + wr), "read_bytes": round(rd),
               "write_bytes": round(wr), "kernel_source_sha256": source_digest(ATTN_SOURCE)}
        print(TRAFFIC_TAG + json.dumps(rec))


MFMA_TAG = "bench-mfma: "
N_CU, N_SIMD, N_XCD = 256, 1024, 8


def sq_summary(csv_path: str) -> None:
    """Per kernel (averaged over its dispatches): the clock from GRBM_GUI_ACTIVE
    (counted on each of the 8 XCDs, so divided by 8) over the dispatch's
    duration; MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (cycles x 1024 SIMDs);
    VALU busy = SQ_ACTIVE_INST_VALU / (cycles x 256 CUs); co-execution =
    SQ_VALU_MFMA_COEXEC_CYCLES / (cycles x 1024 SIMDs); instruction counts per
    dispatch. The attention kernels' figures are tagged with the SHA-256 of
    their source for the bench line."""
    import csv
    rows: dict = {}
    for r in csv.DictReader(open(csv_path)):
        key = (r["Kernel_Name"], r["Dispatch_Id"])
        d = rows.setdefault(key, {"ns": int(r["End_Timestamp"]) - int(r["Start_Timestamp"])})
        d[r["Counter_Name"]] = float(r["Counter_Value"])
    per: dict = {}
    for (name, _), d in rows.items():
        if "ttv::" in name:   # the library's kernels only
            per.setdefault(name, []).append(d)
    print(f"{'kernel':80s} {'n':>3s} {'us':>8s} {'GHz':>5s} {'MFMA%':>6s} {'VALU%':>6s} {'coex%':>6s} "
          f"{'VALU/disp':>10s} {'MFMA/disp':>10s}")
    attn = None
    for name, ds in sorted(per.items(), key=lambda kv: -sum(x["ns"] for x in kv[1])):
        n = len(ds)

        def avg(k):
            return sum(x.get(k, 0.0) for x in ds) / n
        ns = avg("ns")
        cyc = avg("GRBM_GUI_ACTIVE") / N_XCD
        if cyc <= 0 or ns <= 0:
            continue
        mf = 100 * avg("SQ_VALU_MFMA_BUSY_CYCLES") / (cyc * N_SIMD)
        va = 100 * avg("SQ_ACTIVE_INST_VALU") / (cyc * N_CU)
        co = 100 * avg("SQ_VALU_MFMA_COEXEC_CYCLES") / (cyc * N_SIMD)
        print(f"{name[:80]:80s} {n:3d} {ns / 1e3:8.1f} {cyc / ns:5.2f} {mf:6.1f} {va:6.1f} {co:6.1f} "
              f"{avg('SQ_INSTS_VALU'):10.3g} {avg('SQ_INSTS_MFMA'):10.3g}")
        if is_attention_kernel(name) and "merge_kernel" not in name and (attn is None or ns > attn[1]):
            attn = (name, ns, mf, va, co)
    # every counter of the two busiest kernels, per dispatch
    for name, ds in sorted(per.items(), key=lambda kv: -sum(x["ns"] for x in kv[1]))[:2]:
        keys = sorted(k for k in ds[0] if k != "ns")
        print(f"  {name[:60]}: " + ", ".join(f"{k} {sum(x.get(k, 0.0) for x in ds) / len(ds):.4g}" for k in keys))
    if attn is not None:
        print(MFMA_TAG + json.dumps({"kernel": attn[0], "mfma_busy_pct": round(attn[2], 1),
                                     "valu_busy_pct": round(attn[3], 1), "coexec_pct": round(attn[4], 1),
                                     "kernel_source_sha256": source_digest(ATTN_SOURCE)}))


def trace_summary(csv_path: str) -> None:
    """The library's kernels (namespace ttv) of a rocprofv3 kernel_stats.csv,
    slowest total first."""
    import csv
    print(f"{'kernel':82s} {'calls':>6s} {'avg us':>9s} {'min us':>9s} {'max us':>9s} {'total ms':>9s}")
    rows = [r for r in csv.DictReader(open(csv_path)) if "ttv::" in r["Name"]]
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        print(f"{r['Name'][:82]:82s} {int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:9.1f} "
              f"{float(r['MinNs']) / 1e3:9.1f} {float(r['MaxNs']) / 1e3:9.1f} "
              f"{float(r['TotalDurationNs']) / 1e6:9.2f}")


def recorded(path: str, tag: str):
    """The tagged record of a counter summary under profiles/, or None when the
    file is absent or the attention source has changed since the counters
    were taken."""
    try:
        with open(path) as f:
            for line in f:
                if line.startswith(tag):
                    rec = json.loads(line[len(tag):])
                    if rec.get("kernel_source_sha256") == source_digest(ATTN_SOURCE):
                        return rec
    except OSError:
        pass
    return None


def torch_int16():
    import torch
    return torch.int16


def main():
    args = parse()
    if args.pmc_summary:
        pmc_summary(args.pmc_summary[0], args.pmc_summary[1], args.calib_mib)
        return
    if args.sq_summary:
        sq_summary(args.sq_summary)
        return
    if args.trace_summary:
        trace_summary(args.trace_summary)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        if int(os.environ.get("RANK", "0")) == 0:
            print("bench.py measures one GPU: the verify path runs on a single MI355X, so --gpus must be 1",
                  file=sys.stderr)
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
    attn_all = sorted(e0.elapsed_time(e1) for e0, e1 in evs)
    attn_ms = sum(attn_all) / len(attn_all)
    # per-step durations (a further pass, events around each whole step):
    # median and spread next to the block-timed mean
    sevs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    for e0, e1 in sevs:
        e0.record()
        step()
        e1.record()
    torch.cuda.synchronize()
    step_all = sorted(e0.elapsed_time(e1) for e0, e1 in sevs)

    def quantiles(xs):
        def q(f):
            return xs[min(len(xs) - 1, int(round(f * (len(xs) - 1))))]
        return {"median": round(q(0.5), 4), "p10": round(q(0.1), 4), "p90": round(q(0.9), 4),
                "min": round(xs[0], 4), "max": round(xs[-1], 4)}

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
            "us_quantiles": {k: round(v * 1e3, 2) for k, v in quantiles(attn_all).items()},
        }
    }

    # a sliding-window layer of the same round (the pages' 1,024-token window):
    # node i reads the keys past P + i - 1024, i.e. the last 1,023 history rows
    # of every sequence plus its block; algorithmic bytes count those rows once
    W_SLIDE = 1024
    if not args.no_window:
        wws = torch.zeros(ttv.tree_verify_attention_window_ws(batch, spec.Hq, layers[0], spec.q_dtype, W_SLIDE),
                          dtype=torch.uint8, device=dev)
        ttv.tree_verify_attention_window(batch, qs[0], layers[0], anc, scale, W_SLIDE, out, wws)
        wev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(20)]
        torch.cuda.synchronize()
        for i, (e0, e1) in enumerate(wev):
            e0.record()
            ttv.tree_verify_attention_window(batch, qs[i % L], layers[i % L], anc, scale, W_SLIDE, out, wws)
            e1.record()
        torch.cuda.synchronize()
        win_ms = sorted(e0.elapsed_time(e1) for e0, e1 in wev)[len(wev) // 2]
        T_b = np.diff(spec.node_off)
        win_rows = int(np.sum(np.minimum(spec.hist_len, W_SLIDE - 1) + T_b))
        wbytes = (win_rows * spec.Hkv * kv_row_bytes(spec)
                  + spec.n_nodes * spec.Hq * spec.D * ((2 if spec.q_dtype == "bf16" else 4) + 4))
        kernels["tree_verify_attention_window1024"] = {
            "median_us": round(win_ms * 1e3, 2), "bytes": wbytes, "GBps": round(wbytes / (win_ms / 1e3) / 1e9, 1),
            "frac_hbm": round(wbytes / (win_ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
            "what": f"one layer of the round under a {W_SLIDE}-token sliding window (median of 20 launches)",
        }
        print(f"[bench] sliding-window layer (W={W_SLIDE}) {win_ms * 1e3:.1f} us "
              f"({kernels['tree_verify_attention_window1024']['GBps']} GB/s)", file=sys.stderr, flush=True)
        del wws

    # sampled selection (temperature 1, top-k 20, top-p 0.95, one uniform per
    # node): the temperature > 0 form of the argmax step, timed on its own
    n_rows, V = logits.shape
    uni = torch.rand(n_rows, dtype=torch.float32, device=dev, generator=torch.Generator(device=dev).manual_seed(9))
    s_out = torch.empty(n_rows, dtype=torch.int32, device=dev)
    s_ws = torch.empty(ttv.vocab_sample_ws(n_rows, V, 20), dtype=torch.uint8, device=dev)
    ttv.vocab_sample(logits, uni, s_out, s_ws, 1.0, 20, 0.95)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(20):
        ttv.vocab_sample(logits, uni, s_out, s_ws, 1.0, 20, 0.95)
    e1.record()
    torch.cuda.synchronize()
    samp_ms = e0.elapsed_time(e1) / 20
    sbytes = n_rows * V * 4
    kernels["vocab_sample"] = {
        "avg_us": round(samp_ms * 1e3, 2), "bytes": sbytes, "GBps": round(sbytes / (samp_ms / 1e3) / 1e9, 1),
        "frac_hbm": round(sbytes / (samp_ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
        "what": f"{n_rows} x {V} logits, temperature 1, top-k 20, top-p 0.95 (both passes)",
    }
    print(f"[bench] sampled selection {samp_ms * 1e3:.1f} us ({kernels['vocab_sample']['GBps']} GB/s)",
          file=sys.stderr, flush=True)

    # draft tree construction (the step before the mask): per sequence, 8
    # depths of top-4 confidence branching over the drafter's rows, then the
    # 16-node rerank; the drafter's rows are synthetic N(0, 2^2)
    Bd, kd, depths_d, nd = batch.B, 4, 8, 16
    gen_d = torch.Generator(device=dev).manual_seed(11)
    d_rows = [torch.randn(Bd, 1 if d == 0 else kd, V, device=dev, generator=gen_d) * 2.0 for d in range(depths_d)]
    d_table = ttv.DraftTable(Bd, kd, kd + (depths_d - 1) * kd * kd, device=dev)
    d_ws = torch.empty(ttv.draft_tree_expand_ws(Bd * kd, V, kd), dtype=torch.uint8, device=dev)
    d_st = torch.zeros(1, dtype=torch.int32, device=dev)
    d_root = torch.zeros(Bd, dtype=torch.int32, device=dev)
    d_parent = torch.empty(Bd * nd, dtype=torch.int32, device=dev)
    d_token = torch.empty(Bd * nd, dtype=torch.int32, device=dev)

    def build_draft():
        for d in range(depths_d):
            ttv.draft_tree_expand(d_table, d + 1, d_rows[d], d_st, d_ws)
        ttv.draft_tree_select(d_table, nd, d_root, d_parent, d_token, d_st)

    build_draft()
    torch.cuda.synchronize()
    assert int(d_st.item()) == 0, "draft tree status"
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(20):
        build_draft()
    e1.record()
    torch.cuda.synchronize()
    draft_ms = e0.elapsed_time(e1) / 20
    dbytes = sum(r.numel() for r in d_rows) * 4
    kernels["draft_tree"] = {
        "avg_us": round(draft_ms * 1e3, 2), "bytes": dbytes, "GBps": round(dbytes / (draft_ms / 1e3) / 1e9, 1),
        "frac_hbm": round(dbytes / (draft_ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
        "what": f"{Bd} trees of {nd} nodes: {depths_d} expansions of top-{kd} over {V}-logit drafter rows "
                f"(1 row, then {kd} per sequence) + rerank",
    }
    print(f"[bench] draft tree {draft_ms * 1e3:.1f} us ({kernels['draft_tree']['GBps']} GB/s)",
          file=sys.stderr, flush=True)
    del d_rows

    # the argmax fused with the LM-head projection (logits never written):
    # the pages' head, 248,320 vocabulary rows of a 5,120-wide hidden state,
    # bf16 synthetic weights, for this round's nodes and for one 16-node tree
    H_lm = 5120
    gen_lm = torch.Generator(device=dev).manual_seed(12)
    w_lm = (torch.randn(V, H_lm, device=dev, generator=gen_lm) * (1.0 / H_lm ** 0.5)).to(torch.bfloat16)
    for n_lm in sorted({int(batch.n_nodes), 16}):
        x_lm = torch.randn(n_lm, H_lm, device=dev, generator=gen_lm).to(torch.bfloat16)
        o_lm = torch.empty(n_lm, dtype=torch.int32, device=dev)
        ws_lm = torch.empty(ttv.lm_head_argmax_ws(n_lm, V), dtype=torch.uint8, device=dev)
        ttv.lm_head_argmax(x_lm, w_lm, o_lm, ws_lm)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(10):
            ttv.lm_head_argmax(x_lm, w_lm, o_lm, ws_lm)
        e1.record()
        torch.cuda.synchronize()
        lm_ms = e0.elapsed_time(e1) / 10
        lbytes = V * H_lm * 2 + n_lm * H_lm * 2
        lflops = 2 * n_lm * V * H_lm
        kernels[f"lm_head_argmax_n{n_lm}"] = {
            "avg_us": round(lm_ms * 1e3, 2), "bytes": lbytes, "GBps": round(lbytes / (lm_ms / 1e3) / 1e9, 1),
            "frac_hbm": round(lbytes / (lm_ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4), "flops": lflops,
            "TFLOPs": round(lflops / (lm_ms / 1e3) / 1e12, 1),
            "what": f"{n_lm} nodes x {V} x {H_lm} bf16 head, fused argmax (main + reduce launches)",
        }
        print(f"[bench] lm head + argmax, {n_lm} nodes: {lm_ms * 1e3:.1f} us "
              f"({kernels[f'lm_head_argmax_n{n_lm}']['GBps']} GB/s)", file=sys.stderr, flush=True)
        del x_lm
    del w_lm
    # the same over the pages' 4-bit head (codes + a bf16 scale and bias per
    # 64-element group: 635.7 + 39.7 + 39.7 MB), synthetic packed codes
    G_lm = H_lm // 64
    wq_lm = torch.randint(-2 ** 31, 2 ** 31 - 1, (V, H_lm // 8), dtype=torch.int32, device=dev, generator=gen_lm)
    sc_lm = (torch.rand(G_lm, V, device=dev, generator=gen_lm) + 0.5) / (4.6 * H_lm ** 0.5)
    sb_lm = torch.stack([sc_lm, -7.5 * sc_lm], dim=2).to(torch.bfloat16).contiguous()
    for n_lm in sorted({int(batch.n_nodes), 16}):
        x_lm = torch.randn(n_lm, H_lm, device=dev, generator=gen_lm).to(torch.bfloat16)
        o_lm = torch.empty(n_lm, dtype=torch.int32, device=dev)
        ws_lm = torch.empty(ttv.lm_head_q4_argmax_ws(n_lm, V, H_lm), dtype=torch.uint8, device=dev)
        ttv.lm_head_q4_argmax(x_lm, wq_lm, sb_lm, o_lm, ws_lm)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(10):
            ttv.lm_head_q4_argmax(x_lm, wq_lm, sb_lm, o_lm, ws_lm)
        e1.record()
        torch.cuda.synchronize()
        lm_ms = e0.elapsed_time(e1) / 10
        lbytes = V * H_lm // 2 + G_lm * V * 4 + n_lm * H_lm * 2
        lflops = 2 * n_lm * V * H_lm
        kernels[f"lm_head_q4_argmax_n{n_lm}"] = {
            "avg_us": round(lm_ms * 1e3, 2), "bytes": lbytes, "GBps": round(lbytes / (lm_ms / 1e3) / 1e9, 1),
            "frac_hbm": round(lbytes / (lm_ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4), "flops": lflops,
            "TFLOPs": round(lflops / (lm_ms / 1e3) / 1e12, 1),
            "what": f"{n_lm} nodes x {V} x {H_lm} 4-bit head (group 64, bf16 scale/bias), fused argmax",
        }
        print(f"[bench] 4-bit lm head + argmax, {n_lm} nodes: {lm_ms * 1e3:.1f} us "
              f"({kernels[f'lm_head_q4_argmax_n{n_lm}']['GBps']} GB/s)", file=sys.stderr, flush=True)
        del x_lm
    del wq_lm, sb_lm

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
        # the same take of a 50%-scattered selection: half of every sequence's
        # live rows, chosen at random (seeded), in increasing order
        rng = np.random.default_rng(17)
        half = torch.empty(B, cap, dtype=torch.int32, device=dev)
        half_len = np.zeros(B, np.int32)
        for b in range(B):
            keep = np.sort(rng.choice(int(live[b]), size=int(live[b]) // 2, replace=False)).astype(np.int32)
            half[b, :len(keep)] = torch.from_numpy(keep).to(dev)
            half_len[b] = len(keep)
        half_len_d = torch.from_numpy(half_len).to(dev)
        ttv.kv_gather_positions(layers, dst_layers, half, half_len_d, live, st, gws)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.take_reps):
            ttv.kv_gather_positions(layers, dst_layers, half, half_len_d, live, st, gws)
        e1.record()
        torch.cuda.synchronize()
        half_ms = e0.elapsed_time(e1) / args.take_reps
        hrows = int(half_len.sum())
        hbytes = 2 * hrows * spec.Hkv * kv_row_bytes(spec) * L + hrows * 4 * 2
        kernels["kv_gather_positions_take_scatter50"] = {
            "avg_us": round(half_ms * 1e3, 1), "bytes": hbytes, "GBps": round(hbytes / (half_ms / 1e3) / 1e9, 1),
            "frac_hbm": round(hbytes / (half_ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
            "what": "out-of-place take of a random half of every sequence's live rows, all layers",
        }
        print(f"[bench] 50%-scattered take {half_ms:.3f} ms "
              f"({kernels['kv_gather_positions_take_scatter50']['GBps']} GB/s)", file=sys.stderr, flush=True)
        del half
        del dst_caches, dst_layers
        # the practically reachable ceiling for a read+write stream: a plain
        # device copy of 4 GiB (torch's copy kernel), bytes read + written
        a = torch.empty(4 << 30, dtype=torch.uint8, device=dev).fill_(1)
        b2 = torch.empty_like(a)
        b2.copy_(a)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(5):
            b2.copy_(a)
        e1.record()
        torch.cuda.synchronize()
        copy_ms = e0.elapsed_time(e1) / 5
        kernels["plain_copy_4GiB"] = {
            "avg_us": round(copy_ms * 1e3, 1), "bytes": 2 * (4 << 30),
            "GBps": round(2 * (4 << 30) / (copy_ms / 1e3) / 1e9, 1),
            "frac_hbm": round(2 * (4 << 30) / (copy_ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
            "what": "device-to-device copy of 4 GiB (read + write bytes): the reachable ceiling for the take",
        }
        print(f"[bench] plain copy {kernels['plain_copy_4GiB']['GBps']} GB/s", file=sys.stderr, flush=True)
        del a, b2
    assert int(st.item()) == 0, "device status"

    # the in-place rollback of the timed step on its own: the rows it moves
    # (every row from the first non-identity selection entry on, all layers
    # and heads, read and written) and its time
    ttv.kv_gather_positions(layers, None, sel, sel_len, live, st, gws)
    torch.cuda.synchronize()
    pl_h, ph_h = plen.cpu().numpy(), path.cpu().numpy()
    moved_rows = 0
    for b in range(B):
        pth = ph_h[b, :pl_h[b]]
        j0 = next((k for k in range(len(pth)) if pth[k] != k), len(pth))
        moved_rows += len(pth) - j0
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(20):
        ttv.kv_gather_positions(layers, None, sel, sel_len, live, st, gws)
    e1.record()
    torch.cuda.synchronize()
    kernels["kv_gather_positions_rollback"] = {
        "avg_us": round(e0.elapsed_time(e1) / 20 * 1e3, 2),
        "bytes_moved": 2 * moved_rows * spec.Hkv * kv_row_bytes(spec) * L,
        "rows_moved_per_layer_and_head": moved_rows,
        "what": "in-place rollback of the timed round (validate + finalize + compact launches), all layers",
    }

    small = None
    if not args.no_small:
        print("[bench] timing the tiny, chain and 16-layer int8 rounds", file=sys.stderr, flush=True)
        small = small_rounds(dev)
        for k, r in small.items():
            if "us_per_step" in r:
                print(f"[bench] {k}: {r['us_per_step']} us/step, {r['nodes_per_s']} nodes/s "
                      f"(graph replay {r['us_per_step_graph']} us/step)", file=sys.stderr, flush=True)
        print(f"[bench] attention T4/T1 {small['verify_cost_ratio']['T4_over_T1']}, "
              f"T8/T1 {small['verify_cost_ratio']['T8_over_T1']}", file=sys.stderr, flush=True)

    if args.copy_calib_mib > 0:
        a = torch.ones(args.copy_calib_mib << 20, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    cpu = None
    if not args.no_cpu:
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        cpu = cpu_baseline(spec, caches, qs, logits, min(args.cpu_heads, spec.Hkv), min(args.cpu_seqs, B))

    # counter figures recorded for this workload (None once the attention
    # source differs from the one they were taken on)
    traffic = recorded(profile_file(args.config, "traffic"), TRAFFIC_TAG)
    mfma = recorded(profile_file(args.config, "mfma_busy"), MFMA_TAG)
    if mfma:
        kernels["tree_verify_attention"].update(
            {"mfma_busy": round(mfma["mfma_busy_pct"] / 100, 4), "valu_busy": round(mfma["valu_busy_pct"] / 100, 4),
             "mfma_valu_coexec": round(mfma["coexec_pct"] / 100, 4), "counted_kernel": mfma["kernel"]})
    res = {
        "metric": "verified tree nodes/sec + achieved HBM GB/s (verify attn, KV gather) on 1 MI355X",
        "value": round(nodes_per_s, 1),
        "unit": "nodes/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "step_ms_quantiles": quantiles(step_all),
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
                     "frac": round(attn_gbs / HBM_PEAK_GBS, 4),
                     "traffic": traffic["traffic_bytes"] if traffic else None,
                     "kernel": "tree_verify_attention",
                     "mfma_busy": round(mfma["mfma_busy_pct"] / 100, 4) if mfma else None},
        "cpu_baseline": cpu,
        "kernels": kernels,
        "other_rounds": small,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
