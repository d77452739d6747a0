"""Oracle implementation (test infrastructure only; see the package header).

Sources, cited by page title and section:
  [I1204] mlxcel issue #1204, "perf(speculative): draft a tree instead of a
          chain ..." -- sections "What this needs", "Increment 1 landed on a
          branch: topology, mask, walk", "The rollback constraint, which
          decides feasibility", "Redirection ...", "Increment 3: the mask is
          now the shape a forward actually takes".
  [PR1212] mlxcel PR #1212, "feat(speculative): draft and verify a token
          tree, behind a flag, default off" -- its commit messages: the
          topology/mask/walk commit, the gather_positions commit, the commit
          widening the gather to every sequence-axis buffer, the history-mask
          commit, the Gemma 4 tree-verify commit, the verify_finalize_tree
          commit, the gather_within_tail commit, the rollback-to-path commit.
  [I1185] mlxcel issue #1185, "cut the MTP drafter's per-step cost" --
          "Proposed work" (Phase 2a: fuse the LM-head projection and the
          argmax).
  [S728]  splash issue #728, "Experiment: qualify shared-prefix tree
          verification and conservative admission" -- "What it does",
          "Results", "Earlier controlled experiments".
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "decode_bf16",
    "decode_fp16",
    "decode_kv",
    "validate_parent",
    "ancestor_sets",
    "ancestor_bits",
    "node_depths",
    "additive_mask_with_history",
    "sliding_mask_from_caller",
    "visible_keys",
    "attention_rows",
    "tree_verify_attention",
    "tree_verify_attention_dense",
    "vocab_argmax",
    "vocab_sample",
    "lm_head_logits",
    "lm_head_argmax",
    "lm_head_q4_weight",
    "lm_head_q4_logits",
    "lm_head_q4_argmax",
    "tree_accept_walk",
    "draft_tree_new",
    "draft_tree_expand",
    "draft_tree_select",
    "draft_tree",
    "rollback_selection",
    "gather_positions",
    "gather_layer",
    "gather_within_tail",
    "verify_round",
]

MASKED = -1e9  # blocking value of the additive mask ([PR1212] Gemma 4 tree-verify commit)


# ----------------------------------------------------------------------------
# Storage decoding (plain format definitions).
# ----------------------------------------------------------------------------

def decode_bf16(bits) -> np.ndarray:
    """bf16 bit pattern -> float64: the pattern is the top half of an fp32."""
    b = np.asarray(bits).view(np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def decode_fp16(x) -> np.ndarray:
    """IEEE binary16 -> float64 (exact)."""
    return np.asarray(x).view(np.float16).astype(np.float64)


def decode_kv(buf, dtype: str, scale=None) -> np.ndarray:
    """Cache values as float64. int8 codes are dequantised with their per-token
    fp16 scale: value = code * scale ([PR1212] gather_positions commit: Int8
    keeps a per-token scale sidecar on the sequence axis)."""
    if dtype == "f32":
        return np.asarray(buf, dtype=np.float64)
    if dtype == "bf16":
        return decode_bf16(buf)
    if dtype == "i8":
        return np.asarray(buf, dtype=np.int8).astype(np.float64) * decode_fp16(scale)[..., None]
    raise ValueError(dtype)


# ----------------------------------------------------------------------------
# Step 1: ancestor mask.
# ----------------------------------------------------------------------------

def validate_parent(parent) -> None:
    """A draft tree lists its nodes in topological order: node 0 is the root
    (parent -1) and every other node's parent precedes it ([I1204] "Increment
    1": DraftTree keeps parents[i] < i)."""
    for i, p in enumerate(parent):
        p = int(p)
        if i == 0 and p != -1:
            raise ValueError("node 0 must be the root (parent -1)")
        if i > 0 and not (0 <= p < i):
            raise ValueError(f"parent[{i}] = {p} is not an earlier node")


def ancestor_sets(parent) -> list:
    """anc(i) = {i} plus every node on the parent chain from i up to the root,
    found by following the chain explicitly."""
    validate_parent(parent)
    out = []
    for i in range(len(parent)):
        s = set()
        j = i
        while j != -1:
            s.add(j)
            j = int(parent[j])
        out.append(frozenset(s))
    return out


def ancestor_bits(parent) -> np.ndarray:
    """uint64 per node: bit j set iff block node j is in anc(i) (T <= 64)."""
    if len(parent) > 64:
        raise ValueError("more than 64 nodes")
    out = np.zeros(len(parent), dtype=np.uint64)
    for i, s in enumerate(ancestor_sets(parent)):
        w = 0
        for j in s:
            w |= 1 << j
        out[i] = np.uint64(w)
    return out


def node_depths(parent) -> np.ndarray:
    """Number of proper ancestors of each node (root depth 0)."""
    return np.asarray([len(s) - 1 for s in ancestor_sets(parent)], dtype=np.int32)


def additive_mask_with_history(parent, offset: int, masked: float = MASKED) -> np.ndarray:
    """[T, offset + T] float32 additive mask ([I1204] "Increment 3"; [PR1212]
    history-mask commit): query row q sits at logical position q + offset; the
    first ``offset`` columns are the cached history every node attends in
    full; block column offset + j is open (0) iff j is an ancestor of q or q
    itself, and carries ``masked`` otherwise (so siblings never see each
    other). The blocking value is -1e9 rather than -inf ([PR1212] Gemma 4
    tree-verify commit)."""
    T = len(parent)
    m = np.full((T, offset + T), np.float32(masked), dtype=np.float32)
    m[:, :offset] = 0.0
    for q, s in enumerate(ancestor_sets(parent)):
        for j in s:
            m[q, offset + j] = 0.0
    return m


def sliding_mask_from_caller(caller, offset: int, window: int, masked: float = MASKED) -> np.ndarray:
    """The sliding-window layers' mask ([PR1212] the commit intersecting the
    caller mask with the sliding band, and the commit that pulls it into
    sliding_mask_from_caller): the caller's [T, offset + T] additive mask
    intersected (elementwise minimum) with the band that lets query row q,
    at position offset + q, see column c only when offset + q - window < c
    <= offset + q. The pages apply the band only where the two can disagree
    (sliding live length + block length > window); below that the caller
    mask comes back untouched, which the minimum also gives, since the band
    is then all open."""
    caller = np.asarray(caller, dtype=np.float32)
    T, S = caller.shape
    if offset + T <= window:
        return caller.copy()
    q = np.arange(T)[:, None] + offset
    c = np.arange(S)[None, :]
    band = np.where((c > q - window) & (c <= q), np.float32(0.0), np.float32(masked)).astype(np.float32)
    return np.minimum(caller, band)


# ----------------------------------------------------------------------------
# Step 2: tree-masked GQA verify attention.
# ----------------------------------------------------------------------------

def visible_keys(P: int, anc) -> np.ndarray:
    """Cache rows a node attends: the whole prefix [0, P) and the block rows
    P + a for a in anc(i). Block node i's K/V row sits at P + i because the
    verify block is appended in topological order ([PR1212] rollback-to-path
    commit)."""
    return np.concatenate([np.arange(P), P + np.asarray(sorted(anc), dtype=np.int64)]).astype(np.int64)


def attention_rows(qrows, K, V, keys, softmax_scale: float) -> np.ndarray:
    """softmax(scale * q . K[keys]) @ V[keys] for each query row, in float64.
    qrows [n, D]; K, V [S, D] already decoded."""
    q = np.asarray(qrows, dtype=np.float64)
    Kk = K[keys]
    Vk = V[keys]
    s = softmax_scale * (q @ Kk.T)               # [n, |keys|]
    s = s - s.max(axis=1, keepdims=True)
    p = np.exp(s)
    p /= p.sum(axis=1, keepdims=True)
    return p @ Vk


def tree_verify_attention(q, layer: dict, node_off, hist_len, parents, softmax_scale: float,
                          q_dtype: str, kv_dtype: str, window: int = 0) -> np.ndarray:
    """Explicit key-set form, batched over sequences ([I1204] "Redirection":
    the nodes are flattened into one sequence and the tree mask hides
    siblings; [PR1212] history-mask commit: full history plus ancestors).

    q: [n_nodes, Hq, D] (float32 or bf16 bits); layer: {'k','v'[, 'k_scale',
    'v_scale']} with [B, Hkv, cap, D] caches; parents: per-sequence parent
    arrays, or None for the causal (linear) reading. GQA: query head h reads
    KV head h // (Hq / Hkv). window > 0: the sliding-window layers' form,
    node i (cache row P + i) keeping only keys c > P + i - window (see
    sliding_mask_from_caller). Returns float64 [n_nodes, Hq, D]."""
    qf = np.asarray(q, dtype=np.float64) if q_dtype == "f32" else decode_bf16(q)
    n, Hq, D = qf.shape
    Hkv = layer["k"].shape[1]
    G = Hq // Hkv
    out = np.zeros((n, Hq, D), dtype=np.float64)
    B = len(hist_len)
    for b in range(B):
        P = int(hist_len[b])
        o0, o1 = int(node_off[b]), int(node_off[b + 1])
        T = o1 - o0
        if T == 0:
            continue
        par = np.arange(-1, T - 1) if parents is None else parents[b]
        sets = ancestor_sets(par)
        for g in range(Hkv):
            K = decode_kv(layer["k"][b, g, : P + T], kv_dtype, None if kv_dtype != "i8" else layer["k_scale"][b, g, : P + T])
            V = decode_kv(layer["v"][b, g, : P + T], kv_dtype, None if kv_dtype != "i8" else layer["v_scale"][b, g, : P + T])
            for i in range(T):
                keys = visible_keys(P, sets[i])
                if window > 0:
                    keys = keys[keys > P + i - window]
                out[o0 + i, g * G:(g + 1) * G] = attention_rows(qf[o0 + i, g * G:(g + 1) * G], K, V, keys, softmax_scale)
    return out


def tree_verify_attention_dense(qf, K, V, mask_add, softmax_scale: float, G: int) -> np.ndarray:
    """Dense form for one sequence: scores over all P + T cache rows plus the
    additive mask, then softmax and V. qf [T, Hq, D] float64; K, V [Hkv, P+T, D]
    float64; mask_add [T, P+T]."""
    T, Hq, D = qf.shape
    out = np.zeros((T, Hq, D), dtype=np.float64)
    for h in range(Hq):
        g = h // G
        s = softmax_scale * (qf[:, h, :] @ K[g].T) + np.asarray(mask_add, dtype=np.float64)
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p /= p.sum(axis=1, keepdims=True)
        out[:, h, :] = p @ V[g]
    return out


# ----------------------------------------------------------------------------
# Step 3: per-node argmax over the vocabulary.
# ----------------------------------------------------------------------------

def vocab_argmax(logits) -> np.ndarray:
    """The target's greedy selection at every node: the index of the row
    maximum, compared in the logits' own fp32 ([I1204] "Increment 1": the
    target emits one argmax per position; [S728] "Results": raw F32 argmax).
    Ties go to the lowest index; -0.0 equals +0.0; a NaN outranks every number
    and the first NaN wins (numpy.argmax semantics)."""
    return np.argmax(np.asarray(logits, dtype=np.float32), axis=-1).astype(np.int32)


def lm_head_logits(hidden_bits, weight_bits) -> np.ndarray:
    """The target's logits at every node from its final hidden state: the LM
    head's projection logits[n, v] = sum_i hidden[n, i] * weight[v, i], with
    bf16 hidden states [N, H] and a bf16 head weight [V, H] (vocabulary rows),
    in float64 ([I1185] "Proposed work", Phase 2a: at temperature 0 the
    vocabulary-wide logits exist only to take their argmax)."""
    X = decode_bf16(hidden_bits)
    W = decode_bf16(weight_bits)
    return X @ W.T


def lm_head_argmax(hidden_bits, weight_bits) -> np.ndarray:
    """The fused projection-plus-argmax of [I1185] Phase 2a: the index of the
    largest logit of lm_head_logits, ties to the lowest index. The fused form
    never writes the logits; its result is this argmax wherever the float32
    accumulation of the projection cannot reorder the top logits."""
    return np.argmax(lm_head_logits(hidden_bits, weight_bits), axis=-1).astype(np.int32)


def lm_head_q4_weight(wq, sb_bits) -> np.ndarray:
    """The LM head stored the way the pages' engine holds it: affine 4-bit
    codes with one 16-bit scale and bias per group of 64 hidden elements
    ([I1185] "The cost model": the borrowed head is weight 635.7 + scales
    39.7 + biases 39.7 MB for 248,320 x 5,120; the "Phase 3 done" comment:
    affine group-64 4-bit). Value = scale * code + bias, code in 0..15.
    Layout (a reading; the pages give sizes, not layouts): wq uint32 [V, H/8]
    with hidden element i in bits 4 (i mod 8) of word i / 8; sb_bits bf16 bit
    patterns [H/64, V, 2] holding (scale, bias) of group g of row v, group-major.
    Returns the float64 weight [V, H]."""
    wq = np.asarray(wq, dtype=np.uint32)
    sb = np.asarray(sb_bits, dtype=np.uint16)
    V, W8 = wq.shape
    H = 8 * W8
    G = H // 64
    assert sb.shape == (G, V, 2)
    code = np.zeros((V, H), dtype=np.float64)
    for j in range(8):
        code[:, j::8] = (wq >> np.uint32(4 * j)) & np.uint32(15)
    scale = np.repeat(decode_bf16(sb[:, :, 0]).T, 64, axis=1)
    bias = np.repeat(decode_bf16(sb[:, :, 1]).T, 64, axis=1)
    return scale * code + bias


def lm_head_q4_logits(hidden_bits, wq, sb_bits) -> np.ndarray:
    """logits[n, v] = sum_i hidden[n, i] * weight[v, i] over the 4-bit head's
    values, in float64."""
    return decode_bf16(hidden_bits) @ lm_head_q4_weight(wq, sb_bits).T


def lm_head_q4_argmax(hidden_bits, wq, sb_bits) -> np.ndarray:
    """The fused projection-plus-argmax over the 4-bit head ([I1185]
    "Proposed work" Phase 2a and its verdict: a quantised-matmul-with-argmax
    kernel): ties to the lowest index."""
    return np.argmax(lm_head_q4_logits(hidden_bits, wq, sb_bits), axis=-1).astype(np.int32)


def vocab_sample(logits, uniforms, uniform_stride: int, temperature: float, top_k: int, top_p: float) -> np.ndarray:
    """The target's sampled selection at every node ([S728] "Historical issue
    and default question", "What it does": for sampled requests each node
    draws from the nucleus-filtered distribution with its own uniform, node n
    taking uniforms[n * uniform_stride], so stride 0 gives every node the same
    uniform; "Results" quotes temperature 1, top-p 0.95, top-k 20).

    Reading of the filter chain (the pages name its parts, not their order):
      1. top-k: the top_k largest logits, compared in fp32, ties to the lower
         index (the argmax convention; -0.0 == +0.0);
      2. z = logit / temperature and p_i = exp(z_i - z_0) / sum_j exp(z_j - z_0)
         over those k, in float64, summed in descending order;
      3. top-p: keep the shortest descending prefix whose cumulative mass C_i
         reaches top_p (C_{k-1} = 1, so some prefix always does);
      4. draw: the first kept i with C_i > u * C_{i*}, where i* ends the
         prefix and u in [0, 1) is the node's uniform (inverse CDF of the
         renormalised prefix).
    A NaN ranks above every number; a row whose top logit is not finite (NaN,
    +inf, or -inf when every logit is -inf) selects that logit's index. top_k = 1, or top_p <= C_0, reduce to the
    argmax."""
    X = np.asarray(logits, dtype=np.float32)
    U = np.asarray(uniforms, dtype=np.float32).reshape(-1)
    n_rows, V = X.shape
    k = int(min(top_k, V))
    # the parameters are fp32 values (as a caller passes them), widened exactly
    temperature = float(np.float32(temperature))
    top_p = float(np.float32(top_p))
    assert k >= 1 and temperature > 0.0
    out = np.zeros(n_rows, np.int32)
    for n in range(n_rows):
        x = X[n].astype(np.float64)
        # descending by value, ties by index: a stable sort of the keys
        # (NaN first, as the largest)
        nan = np.isnan(x)
        order = np.lexsort((np.arange(V), np.where(nan, 0.0, -x), ~nan))[:k]
        top = x[order[0]]
        if np.isnan(top) or np.isinf(top):
            out[n] = order[0]
            continue
        z = x[order] / float(temperature)
        e = np.exp(z - z[0])
        c = np.zeros(k)
        acc = 0.0
        for i in range(k):  # sequential, descending order
            acc += e[i]
            c[i] = acc
        C = c / acc
        i_star = int(np.argmax(C >= float(top_p)))
        u = float(U[n * int(uniform_stride)])
        target = u * C[i_star]
        pick = i_star
        for i in range(i_star + 1):
            if C[i] > target:
                pick = i
                break
        out[n] = order[pick]
    return out


# ----------------------------------------------------------------------------
# Before step 1: growing the draft tree from the drafter's confidence.
# ----------------------------------------------------------------------------
#
# The pages name the choice and its signal, not the procedure: the branches
# go where the drafter is confident (EAGLE-2), which needs the drafter's
# per-step logits beyond their argmax ([I1204] "What this needs", the fourth
# decision); a drafter that does not branch yields a linear tree, and the
# runner-up at an uncertain step is the alternative worth a verify position
# ([PR1212] Drafter::draft_tree commit); one verify holds the draft chain plus
# alternative leaves picked by a top-16 selector, sixteen unique shared-prefix
# candidates ([S728] "What it does", description). The reading taken is the
# published EAGLE-2 procedure (Li et al. 2024, "EAGLE-2: Faster Inference of
# Language Models with Dynamic Draft Trees"), stated in our own terms:
#   * a candidate's score is the log of its path probability, the sum of the
#     drafter's log-softmax at every step from the root;
#   * expansion, one depth at a time: every frontier node's drafter row gives
#     its top_k tokens by logit as children; the next frontier is the top_k
#     of the new candidates by score; the first frontier is the root alone;
#   * rerank: the tree is the root plus the n_nodes - 1 best candidates by
#     score over every depth. A child's score never exceeds its parent's and
#     ties go to the candidate made first (parents are made before children),
#     so the chosen set is closed under parents. Labels follow that rank, which
#     is a topological order.
# Ties among a row's logits go to the lower token index (the argmax order);
# equal scores go to the lower candidate index. Scores are float64.

def draft_tree_new(root_token: int) -> dict:
    """An empty candidate table for one sequence whose committed token (node
    0 of the tree) is root_token; the first frontier is the root alone."""
    return {"root": int(root_token), "token": [], "parent": [], "score": [], "depth": [],
            "frontier": [-1]}


def _log_softmax_row(x32) -> np.ndarray:
    x = np.asarray(x32, dtype=np.float32).astype(np.float64)
    if not np.isfinite(x).all():
        raise ValueError("drafter logits must be finite")
    m = x.max()
    return x - (m + np.log(np.sum(np.exp(x - m))))


def draft_tree_expand(state: dict, rows, top_k: int) -> dict:
    """One depth of confidence branching: rows[f] is the drafter's logit row
    for frontier node f (in frontier order). Each row contributes its top_k
    tokens (fp32 logits, ties to the lower index) as children of that frontier
    node, scored parent score + log-softmax; the new frontier is the top_k of
    this depth's candidates by score (ties to the lower candidate index), best
    first. Mutates and returns state."""
    rows = np.asarray(rows, dtype=np.float32)
    frontier = state["frontier"]
    assert rows.ndim == 2 and rows.shape[0] == len(frontier), "one row per frontier node"
    V = rows.shape[1]
    assert 1 <= top_k <= V
    first = len(state["token"])
    for f, u in enumerate(frontier):
        lp = _log_softmax_row(rows[f])
        base = 0.0 if u < 0 else state["score"][u]
        d = 1 if u < 0 else state["depth"][u] + 1
        # descending by fp32 logit, ties by index: a stable sort of -x
        order = np.argsort(-rows[f], kind="stable")[:top_k]
        for tok in order:
            state["token"].append(int(tok))
            state["parent"].append(int(u))
            state["score"].append(base + float(lp[tok]))
            state["depth"].append(d)
    new = list(range(first, len(state["token"])))
    new.sort(key=lambda c: (-state["score"][c], c))
    state["frontier"] = new[:top_k]
    return state


def draft_tree_select(state: dict, n_nodes: int):
    """Rerank: node 0 is the root; nodes 1..n_nodes-1 are the best candidates
    by score (ties to the lower candidate index), labelled in that order.
    Returns (parent int32 [n], token int32 [n], score float64 [n]); the root's
    parent is -1 and its score 0."""
    n_cand = len(state["token"])
    if n_nodes < 1 or n_nodes - 1 > n_cand:
        raise ValueError(f"{n_nodes} nodes need {n_nodes - 1} candidates, the table holds {n_cand}")
    ranked = sorted(range(n_cand), key=lambda c: (-state["score"][c], c))[: n_nodes - 1]
    label = {c: r + 1 for r, c in enumerate(ranked)}
    parent = np.full(n_nodes, -1, np.int32)
    token = np.zeros(n_nodes, np.int32)
    score = np.zeros(n_nodes, np.float64)
    token[0] = state["root"]
    for c in ranked:
        u = state["parent"][c]
        parent[label[c]] = 0 if u < 0 else label[u]
        token[label[c]] = state["token"][c]
        score[label[c]] = state["score"][c]
    return parent, token, score


def draft_tree(root_token: int, depth_rows, top_k: int, n_nodes: int):
    """The whole construction for one sequence: depth_rows[d] holds the
    drafter's rows for the frontier at depth d + 1 (one row at d = 0, top_k
    rows after). Returns draft_tree_select's result and the state."""
    st = draft_tree_new(root_token)
    for rows in depth_rows:
        draft_tree_expand(st, rows, top_k)
    return draft_tree_select(st, n_nodes) + (st,)


# ----------------------------------------------------------------------------
# Step 4: tree accept walk.
# ----------------------------------------------------------------------------

def tree_accept_walk(parent, token, target_argmax):
    """Start at the root (node 0, the committed token, never compared). At the
    current node, descend to the child whose draft token equals the target's
    selection at the current node; when two children carry that token take
    the lower label and do not fan out ([I1204] "Increment 1"; [S728] "What it
    does"). Stop when no child matches.

    Returns (path, emitted): path lists node ids from 0; accepted = len(path)
    - 1; emitted[k] = target_argmax[path[k]], i.e. accepted + 1 tokens (the
    accepted drafts plus the target's token after the last one)."""
    validate_parent(parent)
    T = len(parent)
    kids = [[] for _ in range(T)]
    for i in range(1, T):
        kids[int(parent[i])].append(i)
    path = [0]
    cur = 0
    while True:
        nxt = None
        for c in kids[cur]:
            if int(token[c]) == int(target_argmax[cur]):
                nxt = c
                break
        if nxt is None:
            break
        path.append(nxt)
        cur = nxt
    emitted = [int(target_argmax[n]) for n in path]
    return path, emitted


# ----------------------------------------------------------------------------
# Step 5: rollback by gather along the sequence axis.
# ----------------------------------------------------------------------------

def rollback_selection(P: int, path) -> np.ndarray:
    """Survivors of a tree round: the whole history [0, P) and the accepted
    path's block rows P + path[k] ([PR1212] rollback-to-path commit: the cache
    gather is handed the accepted nodes as block offsets)."""
    return np.concatenate([np.arange(P, dtype=np.int64), P + np.asarray(path, dtype=np.int64)])


def gather_positions(buf, sel, axis: int) -> np.ndarray:
    """Select and compact a scattered set of positions along the sequence axis
    ([I1204] "Redirection"; [PR1212] gather_positions commit)."""
    return np.take(buf, np.asarray(sel, dtype=np.int64), axis=axis)


def gather_layer(layer: dict, sels, base: dict | None = None) -> dict:
    """Apply per-sequence selections to one layer's cache [B, Hkv, cap, D] and,
    for int8, its scales [B, Hkv, cap] -- every sequence-axis buffer moves
    with its tokens ([PR1212] gather_positions commit and the commit widening
    it). Rows [0, len(sel_b)) of the result hold the survivors; rows beyond
    keep ``base``'s contents (the source itself for an in-place rollback, the
    destination's prior contents for an out-of-place take)."""
    base = layer if base is None else base
    out = {name: np.array(base[name], copy=True) for name in layer}
    for b, sel in enumerate(sels):
        n = len(sel)
        for name in layer:
            if name.endswith("_scale"):
                out[name][b, :, :n] = gather_positions(layer[name][b], sel, axis=1)
            else:
                out[name][b, :, :n, :] = gather_positions(layer[name][b], sel, axis=1)
    return out


def gather_within_tail(layer: dict, live_len, tail_len, kept) -> dict:
    """Rollback confined to the verify block ([PR1212] gather_within_tail
    commit: offsets within the block, only [tail_start, tail_start +
    kept_len) is rewritten, so the cost follows the block and not the
    context). For sequence b, s = live_len[b] - tail_len[b] and row s + j
    takes row s + kept[b][j] of the input, j < len(kept[b]), in every
    sequence-axis buffer (K, V and the int8 scale sidecars); every other row
    is left as it was. The new live length is s + len(kept[b])."""
    out = {name: np.array(layer[name], copy=True) for name in layer}
    for b, kb in enumerate(kept):
        s = int(live_len[b]) - int(tail_len[b])
        src = s + np.asarray(kb, dtype=np.int64)
        dst = s + np.arange(len(src), dtype=np.int64)
        for name in layer:
            out[name][b, :, dst] = layer[name][b, :, src]
    return out


# ----------------------------------------------------------------------------
# One round.
# ----------------------------------------------------------------------------

def verify_round(spec, tensors: dict, softmax_scale: float | None = None) -> dict:
    """mask -> attention (every layer) -> argmax -> walk -> rollback
    selection -> gather, for a workloads.RoundSpec and its host tensors."""
    scale = 1.0 / np.sqrt(spec.D) if softmax_scale is None else softmax_scale
    node_off = spec.node_off
    anc = np.concatenate([ancestor_bits(p) for p in spec.parents]) if spec.B else np.zeros(0, np.uint64)
    depth = np.concatenate([node_depths(p) for p in spec.parents]) if spec.B else np.zeros(0, np.int32)
    outs = [tree_verify_attention(L["q"], L, node_off, spec.hist_len, spec.parents, scale,
                                  spec.q_dtype, spec.kv_dtype) for L in tensors["layers"]]
    am = vocab_argmax(tensors["logits"])
    paths, emitted, sels = [], [], []
    for b in range(spec.B):
        o0, o1 = int(node_off[b]), int(node_off[b + 1])
        path, em = tree_accept_walk(spec.parents[b], spec.tokens[b], am[o0:o1])
        paths.append(path)
        emitted.append(em)
        sels.append(rollback_selection(int(spec.hist_len[b]), path))
    caches = []
    for L in tensors["layers"]:
        kv = {k: v for k, v in L.items() if k != "q"}
        caches.append(gather_layer(kv, sels))
    return {"anc": anc, "depth": depth, "attn": outs, "argmax": am, "paths": paths,
            "emitted": emitted, "sels": sels, "caches": caches}
