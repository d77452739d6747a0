"""Python binding of libttv (token-tree verification on MI355X).

Argument marshalling only: every step runs in the HIP kernels of libttv.so.
torch tensors supply device memory and the current HIP stream; the functions
carry the C ABI names (see include/ttv.h) and raise TTVError on a non-OK
status. There is no CPU fallback: importing this package fails if the library
has not been built.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libttv.so")

TTV_OK, TTV_ERR_INVALID, TTV_ERR_UNSUPPORTED, TTV_ERR_WORKSPACE, TTV_ERR_HIP = range(5)
TTV_DEV_OK, TTV_DEV_BAD_PARENT, TTV_DEV_BAD_SELECTION, TTV_DEV_BAD_LOGITS, TTV_DEV_DRAFT_STATE = 0, 1, 2, 3, 4
TTV_F32, TTV_BF16, TTV_I8 = 0, 1, 2
MAX_NODES = 64
STATIC_SCRATCH_BYTES = 32 << 20
MAX_BATCH = 128

if not os.path.exists(LIB_PATH):
    raise ImportError(f"libttv.so not built ({LIB_PATH}); run __graft_entry__.build() or "
                      "python token_tree_verification_build_amd/build.py")
_lib = ctypes.CDLL(LIB_PATH)

_p = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_sz = ctypes.c_size_t


class TtvBatch(ctypes.Structure):
    _fields_ = [("B", _i32), ("node_off_h", _p), ("hist_len_h", _p), ("node_off_d", _p), ("hist_len_d", _p)]


class TtvKvLayer(ctypes.Structure):
    _fields_ = [("k", _p), ("v", _p), ("k_scale", _p), ("v_scale", _p), ("dtype", _i32), ("Hkv", _i32),
                ("D", _i32), ("cap", _i32)]


def _sig(name, res, args):
    f = getattr(_lib, name)
    f.restype = res
    f.argtypes = args
    return f


_BP = ctypes.POINTER(TtvBatch)
_LP = ctypes.POINTER(TtvKvLayer)
_c = {
    "tree_build_mask": _sig("tree_build_mask", _i32, [_BP, _p, _p, _p, _p, _p]),
    "tree_mask_expand_additive": _sig("tree_mask_expand_additive", _i32, [_BP, _i32, _p, ctypes.c_float, _p, _p]),
    "tree_verify_attention_ws": _sig("tree_verify_attention_ws", _sz, [_BP, _i32, _LP, _i32]),
    "tree_verify_attention": _sig("tree_verify_attention", _i32,
                                  [_BP, _p, _i32, _i32, _LP, _p, ctypes.c_float, _p, _p, _sz, _p]),
    "tree_verify_attention_static": _sig("tree_verify_attention_static", _i32,
                                         [_BP, _p, _i32, _i32, _LP, _p, ctypes.c_float, _p, _p]),
    "tree_verify_attention_window_ws": _sig("tree_verify_attention_window_ws", _sz, [_BP, _i32, _LP, _i32, _i32]),
    "tree_verify_attention_window": _sig("tree_verify_attention_window", _i32,
                                         [_BP, _p, _i32, _i32, _LP, _p, ctypes.c_float, _i32, _p, _p, _sz, _p]),
    "vocab_argmax_ws": _sig("vocab_argmax_ws", _sz, [_i64, _i64]),
    "vocab_argmax": _sig("vocab_argmax", _i32, [_p, _i64, _i64, _i64, _p, _p, _sz, _p]),
    "vocab_sample_ws": _sig("vocab_sample_ws", _sz, [_i64, _i64, _i32]),
    "vocab_sample": _sig("vocab_sample", _i32, [_p, _i64, _i64, _i64, _p, _i64, ctypes.c_float, _i32,
                                                ctypes.c_float, _p, _p, _sz, _p]),
    "tree_accept_walk": _sig("tree_accept_walk", _i32, [_BP, _p, _p, _p, _p, _p, _p, _p, _i32, _p, _p, _p]),
    "kv_gather_positions_ws": _sig("kv_gather_positions_ws", _sz, [_i32]),
    "kv_gather_positions": _sig("kv_gather_positions", _i32,
                                [_LP, _LP, _i32, _i32, _p, _i32, _p, _p, _p, _p, _sz, _p]),
    "kv_can_gather": _sig("kv_can_gather", _i32, [_LP, _i32]),
    "sliding_mask_from_caller": _sig("sliding_mask_from_caller", _i32,
                                     [_p, _i32, _i32, _i32, _i32, ctypes.c_float, _p, _p]),
    "kv_gather_within_tail_ws": _sig("kv_gather_within_tail_ws", _sz, [_i32]),
    "kv_gather_within_tail": _sig("kv_gather_within_tail", _i32,
                                  [_LP, _i32, _i32, _p, _i32, _p, _p, _p, _p, _p, _p, _sz, _p]),
    "kv_can_gather_within_tail": _sig("kv_can_gather_within_tail", _i32, [_LP, _i32, _i32, _p]),
    "draft_tree_expand_ws": _sig("draft_tree_expand_ws", _sz, [_i32, _i64, _i32]),
    "draft_tree_expand": _sig("draft_tree_expand", _i32, [_i32, _i32, _i32, _p, _i64, _i64, _p, _p, _p, _p, _i32,
                                                          _p, _p, _p, _sz, _p]),
    "draft_tree_select": _sig("draft_tree_select", _i32, [_i32, _i32, _p, _p, _p, _p, _p, _i32, _p, _p, _p, _p, _p]),
    "lm_head_argmax_ws": _sig("lm_head_argmax_ws", _sz, [_i64, _i64]),
    "lm_head_argmax": _sig("lm_head_argmax", _i32, [_p, _i64, _i64, _p, _i64, _i64, _i64, _p, _p, _sz, _p]),
    "lm_head_q4_argmax_ws": _sig("lm_head_q4_argmax_ws", _sz, [_i64, _i64, _i64]),
    "lm_head_q4_argmax": _sig("lm_head_q4_argmax", _i32, [_p, _i64, _i64, _p, _p, _i64, _i64, _p, _p, _sz, _p]),
    "ttv_last_error": _sig("ttv_last_error", ctypes.c_char_p, []),
}

EXPORTED = tuple(_c)


class TTVError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = _c["ttv_last_error"]().decode()
        super().__init__(f"{where}: status {status}: {msg}")


def _check(status: int, where: str) -> None:
    if status != TTV_OK:
        raise TTVError(status, where)


def last_error() -> str:
    return _c["ttv_last_error"]().decode()


def _ptr(t) -> int | None:
    if t is None:
        return None
    return t.data_ptr()


def _stream(stream) -> int | None:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _dev(t, dtype=None, name="tensor"):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    return t


# ---------------------------------------------------------------------------
# descriptors
# ---------------------------------------------------------------------------

class Batch:
    """Host + device copies of node_off [B+1] and hist_len [B]."""

    def __init__(self, node_off, hist_len, device="cuda"):
        import torch
        self.node_off_h = np.ascontiguousarray(node_off, dtype=np.int32)
        self.hist_len_h = np.ascontiguousarray(hist_len, dtype=np.int32)
        self.B = len(self.hist_len_h)
        self.node_off_d = torch.from_numpy(self.node_off_h.copy()).to(device)
        self.hist_len_d = torch.from_numpy(self.hist_len_h.copy()).to(device)
        self.c = TtvBatch(self.B, self.node_off_h.ctypes.data, self.hist_len_h.ctypes.data,
                          self.node_off_d.data_ptr(), self.hist_len_d.data_ptr())

    @property
    def n_nodes(self) -> int:
        return int(self.node_off_h[-1])

    def ref(self):
        return ctypes.byref(self.c)


_DT = {"f32": TTV_F32, "bf16": TTV_BF16, "i8": TTV_I8}


class KVLayer:
    """One layer's cache [B, Hkv, cap, D] (+ fp16 scales [B, Hkv, cap] for int8)."""

    def __init__(self, k, v, k_scale=None, v_scale=None):
        import torch
        want = {torch.float32: "f32", torch.bfloat16: "bf16", torch.int8: "i8"}
        if k.dtype not in want or v.dtype != k.dtype or k.shape != v.shape or k.dim() != 4:
            raise ValueError("k and v must be [B, Hkv, cap, D] tensors of one of float32/bfloat16/int8")
        _dev(k, name="k")
        _dev(v, name="v")
        self.dtype = want[k.dtype]
        if self.dtype == "i8":
            for s, n in ((k_scale, "k_scale"), (v_scale, "v_scale")):
                if s is not None:
                    _dev(s, torch.float16, n)
                    if tuple(s.shape) != tuple(k.shape[:3]):
                        raise ValueError(f"{n} must be [B, Hkv, cap]")
        self.k, self.v, self.k_scale, self.v_scale = k, v, k_scale, v_scale
        B, Hkv, cap, D = k.shape
        self.Hkv, self.cap, self.D = Hkv, cap, D
        self.c = TtvKvLayer(k.data_ptr(), v.data_ptr(), _ptr(k_scale), _ptr(v_scale), _DT[self.dtype], Hkv, D, cap)

    def ref(self):
        return ctypes.byref(self.c)


def _layers_array(layers):
    arr = (TtvKvLayer * len(layers))()
    for i, L in enumerate(layers):
        arr[i] = L.c
    return arr


# ---------------------------------------------------------------------------
# the C ABI, one function each
# ---------------------------------------------------------------------------

def tree_build_mask(batch: Batch, parent, anc, depth, dev_status, stream=None):
    import torch
    _dev(parent, torch.int32, "parent")
    _dev(anc, torch.int64, "anc")
    _dev(depth, torch.int32, "depth")
    _dev(dev_status, torch.int32, "dev_status")
    _check(_c["tree_build_mask"](batch.ref(), _ptr(parent), _ptr(anc), _ptr(depth), _ptr(dev_status),
                                 _stream(stream)), "tree_build_mask")


def tree_mask_expand_additive(batch: Batch, b: int, anc, masked: float, out, stream=None):
    import torch
    _dev(anc, torch.int64, "anc")
    _dev(out, torch.float32, "out")
    _check(_c["tree_mask_expand_additive"](batch.ref(), b, _ptr(anc), masked, _ptr(out), _stream(stream)),
           "tree_mask_expand_additive")


def sliding_mask_from_caller(caller, offset: int, window: int, masked: float, out, stream=None):
    """caller, out: float32 device tensors [T, S] (out may be caller)."""
    import torch
    _dev(caller, torch.float32, "caller")
    _dev(out, torch.float32, "out")
    if caller.dim() != 2 or tuple(out.shape) != tuple(caller.shape):
        raise ValueError("caller and out must be [T, S] of one shape")
    T, S = caller.shape
    _check(_c["sliding_mask_from_caller"](_ptr(caller), T, S, offset, window, masked, _ptr(out), _stream(stream)),
           "sliding_mask_from_caller")


def tree_verify_attention_ws(batch: Batch, Hq: int, layer: KVLayer, q_dtype: str) -> int:
    return int(_c["tree_verify_attention_ws"](batch.ref(), Hq, layer.ref(), _DT[q_dtype]))


def tree_verify_attention(batch: Batch, q, layer: KVLayer, anc, softmax_scale: float, out, ws, stream=None):
    """q [n_nodes, Hq, D] float32 or bfloat16; out float32 like q; anc int64 or None (causal);
    ws: uint8 device tensor of at least tree_verify_attention_ws bytes, any contents (the call writes every
    workspace byte it reads)."""
    import torch
    _dev(q, name="q")
    qd = {torch.float32: "f32", torch.bfloat16: "bf16"}[q.dtype]
    _dev(out, torch.float32, "out")
    _dev(anc, torch.int64, "anc")
    _dev(ws, torch.uint8, "ws")
    Hq = q.shape[1]
    _check(_c["tree_verify_attention"](batch.ref(), _ptr(q), _DT[qd], Hq, layer.ref(), _ptr(anc), softmax_scale,
                                       _ptr(out), _ptr(ws), ws.numel() if ws is not None else 0, _stream(stream)),
           "tree_verify_attention")


def tree_verify_attention_static(batch: Batch, q, layer: KVLayer, anc, softmax_scale: float, out, stream=None):
    """tree_verify_attention with the library's static per-device scratch in place of a workspace (allocates
    nothing; calls that overlap on one device race). Raises TTVError (TTV_ERR_UNSUPPORTED) when the call's
    partials exceed STATIC_SCRATCH_BYTES."""
    import torch
    _dev(q, name="q")
    qd = {torch.float32: "f32", torch.bfloat16: "bf16"}[q.dtype]
    _dev(out, torch.float32, "out")
    _dev(anc, torch.int64, "anc")
    _check(_c["tree_verify_attention_static"](batch.ref(), _ptr(q), _DT[qd], q.shape[1], layer.ref(), _ptr(anc),
                                              softmax_scale, _ptr(out), _stream(stream)),
           "tree_verify_attention_static")


def tree_verify_attention_window_ws(batch: Batch, Hq: int, layer: KVLayer, q_dtype: str, window: int) -> int:
    return int(_c["tree_verify_attention_window_ws"](batch.ref(), Hq, layer.ref(), _DT[q_dtype], window))


def tree_verify_attention_window(batch: Batch, q, layer: KVLayer, anc, softmax_scale: float, window: int, out, ws,
                                 stream=None):
    """tree_verify_attention with node i keeping only keys > P + i - window."""
    import torch
    _dev(q, name="q")
    qd = {torch.float32: "f32", torch.bfloat16: "bf16"}[q.dtype]
    _dev(out, torch.float32, "out")
    _dev(anc, torch.int64, "anc")
    _dev(ws, torch.uint8, "ws")
    Hq = q.shape[1]
    _check(_c["tree_verify_attention_window"](batch.ref(), _ptr(q), _DT[qd], Hq, layer.ref(), _ptr(anc),
                                              softmax_scale, window, _ptr(out), _ptr(ws),
                                              ws.numel() if ws is not None else 0, _stream(stream)),
           "tree_verify_attention_window")


def vocab_argmax_ws(n_rows: int, vocab: int) -> int:
    return int(_c["vocab_argmax_ws"](n_rows, vocab))


def vocab_argmax(logits, out_idx, ws=None, n_rows=None, vocab=None, row_stride=None, stream=None):
    """logits: float32 device tensor [n_rows, >= vocab] (row stride from the tensor unless given)."""
    import torch
    if logits.dtype != torch.float32 or not logits.is_cuda or logits.stride(-1) != 1:
        raise ValueError("logits must be a float32 device tensor with unit inner stride")
    n_rows = logits.shape[0] if n_rows is None else n_rows
    vocab = logits.shape[1] if vocab is None else vocab
    row_stride = logits.stride(0) if row_stride is None else row_stride
    _dev(out_idx, torch.int32, "out_idx")
    _check(_c["vocab_argmax"](_ptr(logits), n_rows, vocab, row_stride, _ptr(out_idx), _ptr(ws),
                              ws.numel() if ws is not None else 0, _stream(stream)), "vocab_argmax")


def vocab_sample_ws(n_rows: int, vocab: int, top_k: int) -> int:
    return int(_c["vocab_sample_ws"](n_rows, vocab, top_k))


def vocab_sample(logits, uniforms, out_idx, ws, temperature: float, top_k: int, top_p: float,
                 uniform_stride: int = 1, n_rows=None, vocab=None, row_stride=None, stream=None):
    """logits: float32 device tensor [n_rows, >= vocab]; uniforms: float32 device
    tensor, node n taking uniforms[n * uniform_stride]."""
    import torch
    if logits.dtype != torch.float32 or not logits.is_cuda or logits.stride(-1) != 1:
        raise ValueError("logits must be a float32 device tensor with unit inner stride")
    n_rows = logits.shape[0] if n_rows is None else n_rows
    vocab = logits.shape[1] if vocab is None else vocab
    row_stride = logits.stride(0) if row_stride is None else row_stride
    _dev(uniforms, torch.float32, "uniforms")
    if n_rows > 0 and uniforms.numel() <= (n_rows - 1) * uniform_stride:
        raise ValueError("uniforms holds fewer than (n_rows - 1) * uniform_stride + 1 values")
    _dev(out_idx, torch.int32, "out_idx")
    _check(_c["vocab_sample"](_ptr(logits), n_rows, vocab, row_stride, _ptr(uniforms), uniform_stride,
                              float(temperature), int(top_k), float(top_p), _ptr(out_idx), _ptr(ws),
                              ws.numel() if ws is not None else 0, _stream(stream)), "vocab_sample")


def tree_accept_walk(batch: Batch, parent, token, target_argmax, path, path_len, emitted, dev_status,
                     sel=None, sel_len_out=None, stream=None):
    import torch
    for t, n in ((parent, "parent"), (token, "token"), (target_argmax, "target_argmax"), (path, "path"),
                 (path_len, "path_len"), (emitted, "emitted"), (dev_status, "dev_status"), (sel, "sel"),
                 (sel_len_out, "sel_len_out")):
        _dev(t, torch.int32, n)
    stride = sel.shape[1] if sel is not None else 0
    _check(_c["tree_accept_walk"](batch.ref(), _ptr(parent), _ptr(token), _ptr(target_argmax), _ptr(path),
                                  _ptr(path_len), _ptr(emitted), _ptr(sel), stride, _ptr(sel_len_out),
                                  _ptr(dev_status), _stream(stream)), "tree_accept_walk")


def kv_gather_positions_ws(B: int) -> int:
    return int(_c["kv_gather_positions_ws"](B))


def kv_gather_positions(src_layers, dst_layers, sel, sel_len, live_len_h, dev_status, ws, stream=None):
    """src_layers/dst_layers: lists of KVLayer (dst None = in place). sel int32 [B, stride]."""
    import torch
    _dev(sel, torch.int32, "sel")
    _dev(sel_len, torch.int32, "sel_len")
    _dev(dev_status, torch.int32, "dev_status")
    _dev(ws, None, "ws")
    live = np.ascontiguousarray(live_len_h, dtype=np.int32)
    src = _layers_array(src_layers)
    dst = _layers_array(dst_layers) if dst_layers is not None else None
    B = sel.shape[0]
    _check(_c["kv_gather_positions"](src, dst, len(src_layers), B, _ptr(sel), sel.shape[1], _ptr(sel_len),
                                     live.ctypes.data, _ptr(dev_status), _ptr(ws), ws.numel() * ws.element_size(),
                                     _stream(stream)), "kv_gather_positions")


def kv_can_gather(layers) -> tuple[int, str]:
    arr = _layers_array(layers)
    st = _c["kv_can_gather"](arr, len(layers))
    return st, last_error()


def kv_can_gather_raw(layer_structs) -> tuple[int, str]:
    """Capability query on raw TtvKvLayer structs (no tensors needed)."""
    arr = (TtvKvLayer * len(layer_structs))(*layer_structs)
    st = _c["kv_can_gather"](arr, len(layer_structs))
    return st, last_error()


def kv_gather_within_tail_ws(B: int) -> int:
    return int(_c["kv_gather_within_tail_ws"](B))


def _wrapped_arg(ring_wrapped, B):
    if ring_wrapped is None:
        return None, None
    w = np.ascontiguousarray(ring_wrapped, dtype=np.int32)
    if w.shape != (B,):
        raise ValueError("ring_wrapped must hold one flag per sequence")
    return w, w.ctypes.data


def kv_gather_within_tail(layers, kept, kept_len, live_len_h, tail_len_h, dev_status, ws, ring_wrapped=None,
                          stream=None):
    """In-place rollback confined to each sequence's last tail_len rows.
    kept int32 [B, stride] offsets inside the tail; ring_wrapped: host flags or None."""
    import torch
    _dev(kept, torch.int32, "kept")
    _dev(kept_len, torch.int32, "kept_len")
    _dev(dev_status, torch.int32, "dev_status")
    _dev(ws, None, "ws")
    B = kept.shape[0]
    live = np.ascontiguousarray(live_len_h, dtype=np.int32)
    tail = np.ascontiguousarray(tail_len_h, dtype=np.int32)
    if live.shape != (B,) or tail.shape != (B,):
        raise ValueError("live_len_h and tail_len_h must hold one entry per sequence")
    w, wp = _wrapped_arg(ring_wrapped, B)
    arr = _layers_array(layers)
    _check(_c["kv_gather_within_tail"](arr, len(layers), B, _ptr(kept), kept.shape[1], _ptr(kept_len),
                                       live.ctypes.data, tail.ctypes.data, wp, _ptr(dev_status), _ptr(ws),
                                       ws.numel() * ws.element_size(), _stream(stream)), "kv_gather_within_tail")


def kv_can_gather_within_tail(layers, B: int, ring_wrapped=None) -> tuple[int, str]:
    w, wp = _wrapped_arg(ring_wrapped, B)
    arr = _layers_array(layers)
    st = _c["kv_can_gather_within_tail"](arr, len(layers), B, wp)
    return st, last_error()


class DraftTable:
    """Device candidate tables of a batch of draft trees (one per sequence):
    cand_token / cand_parent int32 [B, cap], cand_score float64 [B, cap],
    cand_count int32 [B], frontier int32 [B, top_k]."""

    def __init__(self, B: int, top_k: int, cap: int, device="cuda"):
        import torch
        self.B, self.top_k, self.cap = int(B), int(top_k), int(cap)
        self.cand_token = torch.zeros(B, cap, dtype=torch.int32, device=device)
        self.cand_parent = torch.zeros(B, cap, dtype=torch.int32, device=device)
        self.cand_score = torch.zeros(B, cap, dtype=torch.float64, device=device)
        self.cand_count = torch.zeros(B, dtype=torch.int32, device=device)
        self.frontier = torch.zeros(B, top_k, dtype=torch.int32, device=device)


def draft_tree_expand_ws(n_rows: int, vocab: int, top_k: int) -> int:
    return int(_c["draft_tree_expand_ws"](n_rows, vocab, top_k))


def draft_tree_expand(table: DraftTable, depth: int, logits, status, ws, vocab=None, stream=None):
    """One depth of confidence branching for every sequence. logits: float32
    device tensor [B * F, >= vocab] or [B, F, >= vocab] with unit inner
    stride, F = 1 at depth 1 and top_k after."""
    import torch
    if logits.dtype != torch.float32 or not logits.is_cuda or logits.stride(-1) != 1:
        raise ValueError("logits must be a float32 device tensor with unit inner stride")
    F = 1 if depth == 1 else table.top_k
    B = table.B
    if logits.dim() == 3:
        if logits.shape[0] != B or logits.shape[1] != F:
            raise ValueError(f"logits must be [B={B}, F={F}, V]")
        if B * F == 1:
            row_stride = logits.shape[-1]  # one row: any stride >= vocab
        elif F == 1:
            row_stride = logits.stride(0)
        elif B == 1 or logits.stride(0) == F * logits.stride(1):
            row_stride = logits.stride(1)
        else:
            raise ValueError("logits rows must be evenly spaced")
    elif logits.dim() == 2:
        if logits.shape[0] != B * F:
            raise ValueError(f"logits must hold B * F = {B * F} rows")
        row_stride = logits.stride(0) if B * F > 1 else logits.shape[-1]
    else:
        raise ValueError("logits must be 2-D or 3-D")
    vocab = logits.shape[-1] if vocab is None else vocab
    _dev(status, torch.int32, "status")
    _check(_c["draft_tree_expand"](table.B, int(depth), table.top_k, _ptr(logits), vocab, row_stride,
                                   _ptr(table.cand_token), _ptr(table.cand_parent), _ptr(table.cand_score),
                                   _ptr(table.cand_count), table.cap, _ptr(table.frontier), _ptr(status), _ptr(ws),
                                   ws.numel() if ws is not None else 0, _stream(stream)), "draft_tree_expand")


def draft_tree_select(table: DraftTable, n_nodes: int, root_token, parent, token, status, node_score=None,
                      stream=None):
    """Trees of n_nodes nodes per sequence into parent / token int32 [B * n_nodes]
    (node_off[b] = b * n_nodes); node_score float64 [B * n_nodes] optional."""
    import torch
    _dev(root_token, torch.int32, "root_token")
    _dev(parent, torch.int32, "parent")
    _dev(token, torch.int32, "token")
    _dev(status, torch.int32, "status")
    if parent.numel() < table.B * n_nodes or token.numel() < table.B * n_nodes or root_token.numel() < table.B:
        raise ValueError("parent / token must hold B * n_nodes entries and root_token B")
    if node_score is not None:
        _dev(node_score, torch.float64, "node_score")
        if node_score.numel() < table.B * n_nodes:
            raise ValueError("node_score must hold B * n_nodes entries")
    _check(_c["draft_tree_select"](table.B, int(n_nodes), _ptr(root_token), _ptr(table.cand_token),
                                   _ptr(table.cand_parent), _ptr(table.cand_score), _ptr(table.cand_count), table.cap,
                                   _ptr(parent), _ptr(token), _ptr(node_score), _ptr(status), _stream(stream)),
           "draft_tree_select")


def lm_head_argmax_ws(n_rows: int, vocab: int) -> int:
    return int(_c["lm_head_argmax_ws"](n_rows, vocab))


def lm_head_argmax(hidden, weight, out_idx, ws, stream=None):
    """hidden: bf16 device tensor [N, >= H]; weight: bf16 device tensor
    [V, >= H] (H = hidden.shape[1] unless the views differ), unit inner
    strides; out_idx int32 [N]."""
    import torch
    for t, name in ((hidden, "hidden"), (weight, "weight")):
        if t.dtype != torch.bfloat16 or not t.is_cuda or t.dim() != 2 or t.stride(-1) != 1:
            raise ValueError(f"{name} must be a 2-D bf16 device tensor with unit inner stride")
    if hidden.shape[1] != weight.shape[1]:
        raise ValueError("hidden and weight must share the hidden dimension")
    _dev(out_idx, torch.int32, "out_idx")
    N, H = hidden.shape
    V = weight.shape[0]
    if out_idx.numel() < N:
        raise ValueError("out_idx must hold one index per hidden row")
    hs = hidden.stride(0) if N > 1 else H + (-H) % 8
    wst = weight.stride(0) if V > 1 else H + (-H) % 8
    _check(_c["lm_head_argmax"](_ptr(hidden), N, hs, _ptr(weight), V, H, wst, _ptr(out_idx), _ptr(ws),
                                ws.numel() if ws is not None else 0, _stream(stream)), "lm_head_argmax")


def lm_head_q4_argmax_ws(n_rows: int, vocab: int, hidden_dim: int) -> int:
    return int(_c["lm_head_q4_argmax_ws"](n_rows, vocab, hidden_dim))


def lm_head_q4_argmax(hidden, wq, scale_bias, out_idx, ws, stream=None):
    """hidden: bf16 device tensor [N, >= H]; wq: int32 device tensor
    [V, H / 8] of packed 4-bit codes; scale_bias: bf16 device tensor
    [H / 64, V, 2] of (scale, bias); out_idx int32 [N]."""
    import torch
    if hidden.dtype != torch.bfloat16 or not hidden.is_cuda or hidden.dim() != 2 or hidden.stride(-1) != 1:
        raise ValueError("hidden must be a 2-D bf16 device tensor with unit inner stride")
    _dev(wq, None, "wq")
    _dev(scale_bias, torch.bfloat16, "scale_bias")
    if wq.dtype not in (torch.int32, torch.uint32) or wq.dim() != 2:
        raise ValueError("wq must be a 2-D 32-bit tensor of packed codes")
    N, H = hidden.shape
    V = wq.shape[0]
    if wq.shape[1] * 8 != H or tuple(scale_bias.shape) != (H // 64, V, 2):
        raise ValueError("wq must be [V, H / 8] and scale_bias [H / 64, V, 2] for hidden [N, H]")
    _dev(out_idx, torch.int32, "out_idx")
    if out_idx.numel() < N:
        raise ValueError("out_idx must hold one index per hidden row")
    hs = hidden.stride(0) if N > 1 else H + (-H) % 8
    _check(_c["lm_head_q4_argmax"](_ptr(hidden), N, hs, _ptr(wq), _ptr(scale_bias), V, H, _ptr(out_idx), _ptr(ws),
                                   ws.numel() if ws is not None else 0, _stream(stream)), "lm_head_q4_argmax")
