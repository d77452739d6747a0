"""CPU-side checks of the C ABI: the library loads, exports every symbol the
header declares, and its host-side validation refuses malformed calls before
anything is launched (no call here reaches a kernel launch)."""

import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ttv.h")

ttv = pytest.importorskip("token_tree_verification_build_amd",
                          reason="libttv.so not built (run __graft_entry__.build())")
C = ttv._c
FAKE = 0x10000  # never dereferenced: every call below fails validation on the host


def header_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^(?:ttv_status|size_t|const char\*)\s+(\w+)\s*\(", text, re.M)))


def test_exports_every_declared_symbol():
    names = header_functions()
    assert len(names) >= 11
    lib = ctypes.CDLL(ttv.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(ttv.EXPORTED)


def batch(node_off, hist, dev=True):
    no = np.ascontiguousarray(node_off, dtype=np.int32)
    hl = np.ascontiguousarray(hist, dtype=np.int32)
    b = ttv.TtvBatch(len(hl), no.ctypes.data, hl.ctypes.data, FAKE if dev else None, FAKE if dev else None)
    return b, (no, hl)


def layer(dtype=ttv.TTV_BF16, Hkv=8, D=128, cap=4096, scales=False):
    s = FAKE if scales else None
    return ttv.TtvKvLayer(FAKE, FAKE, s, s, dtype, Hkv, D, cap)


def test_last_error_empty_after_ok_query():
    b, keep = batch([0, 4], [10])
    assert C["tree_verify_attention_ws"](ctypes.byref(b), 40, ctypes.byref(layer()), ttv.TTV_BF16) > 0
    st, msg = ttv.kv_can_gather_raw([layer()])
    assert st == ttv.TTV_OK and msg == ""


def test_mask_rejects_oversized_tree():
    b, keep = batch([0, 65], [0])
    st = C["tree_build_mask"](ctypes.byref(b), FAKE, FAKE, FAKE, FAKE, None)
    assert st == ttv.TTV_ERR_INVALID and "65 nodes" in ttv.last_error()


def test_mask_rejects_bad_offsets_and_batch():
    b, keep = batch([1, 3], [0])
    assert C["tree_build_mask"](ctypes.byref(b), FAKE, FAKE, FAKE, FAKE, None) == ttv.TTV_ERR_INVALID
    b, keep = batch([0, 5, 3], [0, 0])
    assert C["tree_build_mask"](ctypes.byref(b), FAKE, FAKE, FAKE, FAKE, None) == ttv.TTV_ERR_INVALID
    no = np.zeros(ttv.MAX_BATCH + 2, np.int32)
    hl = np.zeros(ttv.MAX_BATCH + 1, np.int32)
    b = ttv.TtvBatch(ttv.MAX_BATCH + 1, no.ctypes.data, hl.ctypes.data, FAKE, FAKE)
    assert C["tree_build_mask"](ctypes.byref(b), FAKE, FAKE, FAKE, FAKE, None) == ttv.TTV_ERR_INVALID
    b, keep = batch([0, 3], [-1])
    assert C["tree_build_mask"](ctypes.byref(b), FAKE, FAKE, FAKE, FAKE, None) == ttv.TTV_ERR_INVALID


def test_mask_null_pointers():
    b, keep = batch([0, 3], [0])
    assert C["tree_build_mask"](ctypes.byref(b), None, FAKE, FAKE, FAKE, None) == ttv.TTV_ERR_INVALID


def _attn(b, Hq, L, q_dtype=ttv.TTV_BF16, ws_bytes=1 << 40):
    return C["tree_verify_attention"](ctypes.byref(b), FAKE, q_dtype, Hq, ctypes.byref(L), None, 0.1, FAKE,
                                      FAKE, ws_bytes, None)


def test_attention_validation():
    b, keep = batch([0, 16], [4096])
    assert _attn(b, 42, layer()) == ttv.TTV_ERR_INVALID            # Hq % Hkv
    assert "multiple" in ttv.last_error()
    assert _attn(b, 40, layer(D=96)) == ttv.TTV_ERR_INVALID        # head dim
    assert _attn(b, 40, layer(cap=4100)) == ttv.TTV_ERR_INVALID    # cap < P + T
    assert "cache holds" in ttv.last_error()
    assert _attn(b, 40, layer(dtype=ttv.TTV_I8, cap=8192)) == ttv.TTV_ERR_UNSUPPORTED   # no scale sidecars
    assert _attn(b, 40, layer(dtype=ttv.TTV_F32, cap=8192)) == ttv.TTV_ERR_UNSUPPORTED  # bf16 q with f32 KV
    assert _attn(b, 40, layer(cap=8192), q_dtype=ttv.TTV_F32) == ttv.TTV_ERR_UNSUPPORTED
    assert _attn(b, 40, layer(cap=8192), ws_bytes=16) == ttv.TTV_ERR_WORKSPACE


def test_attention_ws_sizes():
    L = layer(dtype=ttv.TTV_I8, scales=True, cap=140000)
    b, keep = batch(np.arange(9) * 16, [131072] * 8)
    n = C["tree_verify_attention_ws"](ctypes.byref(b), 40, ctypes.byref(L), ttv.TTV_BF16)
    assert 0 < n < 512 << 20
    bad, keep2 = batch([0, 16], [4096])
    assert C["tree_verify_attention_ws"](ctypes.byref(bad), 41, ctypes.byref(L), ttv.TTV_BF16) == 0


def test_attention_planner_partial_bound():
    """Replays the attention planner on the host over the shapes the merge
    launch must take: every plan keeps a unit's partials within the merge
    workgroup's weight table (the planner refuses a plan that would not, so a
    workspace size of 0 here would mean such a refusal)."""
    hist = [0, 1, 31, 1000, 4096, 10999, 11000, 16384, 50000, 131072]
    n_plans = 0
    for dt, scales in ((ttv.TTV_BF16, False), (ttv.TTV_I8, True)):
        for B in (1, 2, 4):
            for T in (1, 16, 20, 33, 48, 64):
                for P in hist:
                    L = layer(dtype=dt, scales=scales, cap=P + 64)
                    b, keep = batch(np.arange(B + 1) * T, [P] * B)
                    for window in (0, 1024):
                        if window:
                            n = C["tree_verify_attention_window_ws"](ctypes.byref(b), 40, ctypes.byref(L),
                                                                     ttv.TTV_BF16, window)
                        else:
                            n = C["tree_verify_attention_ws"](ctypes.byref(b), 40, ctypes.byref(L), ttv.TTV_BF16)
                        assert n > 0, (dt, B, T, P, window, ttv.last_error())
                        n_plans += 1
    # ragged batches: one long sequence among short ones
    for dt, scales in ((ttv.TTV_BF16, False), (ttv.TTV_I8, True)):
        L = layer(dtype=dt, scales=scales, cap=131072 + 64)
        b, keep = batch([0, 64, 65, 105], [131072, 3, 20000])
        assert C["tree_verify_attention_ws"](ctypes.byref(b), 40, ctypes.byref(L), ttv.TTV_BF16) > 0
    assert n_plans == 2 * 3 * 6 * len(hist) * 2


def test_static_attention_refuses_beyond_its_scratch():
    """The allocation-free attention entry point plans on the host and
    refuses, before any device call, a call whose partials exceed its static
    scratch; the long-context layer fits."""
    from workloads import config4_round, config5_round
    assert ttv.STATIC_SCRATCH_BYTES == 32 << 20
    text = open(HEADER).read()
    assert "#define TTV_STATIC_SCRATCH_BYTES (32u << 20)" in text
    spec = config4_round()
    b, keep = batch(spec.node_off, spec.hist_len)
    L = layer(cap=int(max(spec.hist_len + np.diff(spec.node_off))))
    assert C["tree_verify_attention_ws"](ctypes.byref(b), 40, ctypes.byref(L), ttv.TTV_BF16) > ttv.STATIC_SCRATCH_BYTES
    st = C["tree_verify_attention_static"](ctypes.byref(b), FAKE, ttv.TTV_BF16, 40, ctypes.byref(L), None, 0.1, FAKE,
                                           None)
    assert st == ttv.TTV_ERR_UNSUPPORTED and "static scratch" in ttv.last_error()
    # host validation runs first, as for the workspace form
    bad, keep2 = batch([0, 16], [4096])
    assert C["tree_verify_attention_static"](ctypes.byref(bad), FAKE, ttv.TTV_BF16, 42, ctypes.byref(layer()), None,
                                             0.1, FAKE, None) == ttv.TTV_ERR_INVALID
    spec5 = config5_round(0, [131072] * 8, "tree", L=1)
    b5, keep5 = batch(spec5.node_off, spec5.hist_len)
    L5 = layer(dtype=ttv.TTV_I8, scales=True, cap=131072 + 16)
    assert 0 < C["tree_verify_attention_ws"](ctypes.byref(b5), 40, ctypes.byref(L5), ttv.TTV_BF16) <= \
        ttv.STATIC_SCRATCH_BYTES


def test_argmax_validation():
    f = C["vocab_argmax"]
    assert f(FAKE, 4, 100, 99, FAKE, None, 0, None) == ttv.TTV_ERR_INVALID       # stride < vocab
    assert f(FAKE, 4, 0, 0, FAKE, None, 0, None) == ttv.TTV_ERR_INVALID          # empty vocab
    assert f(FAKE, 0, 10, 10, FAKE, None, 0, None) == ttv.TTV_OK                 # no rows: nothing to do
    need = C["vocab_argmax_ws"](3, 248320)
    assert need > 0
    assert f(FAKE, 3, 248320, 248320, FAKE, FAKE, need - 8, None) == ttv.TTV_ERR_WORKSPACE
    assert C["vocab_argmax_ws"](4096, 1024) == 0


def test_sample_validation():
    f = C["vocab_sample"]
    need = C["vocab_sample_ws"](128, 248320, 20)
    assert need == 128 * 61 * 20 * 8
    ok = (FAKE, 128, 248320, 248320, FAKE, 1, 1.0, 20, 0.95, FAKE, FAKE, need, None)

    def call(**kw):
        a = list(ok)
        names = ["logits", "n_rows", "vocab", "stride", "u", "ustride", "temp", "k", "p", "out", "ws", "wsb", "st"]
        for n, v in kw.items():
            a[names.index(n)] = v
        return f(*a)

    assert call(k=0) == ttv.TTV_ERR_INVALID
    assert call(k=65) == ttv.TTV_ERR_INVALID
    assert call(temp=0.0) == ttv.TTV_ERR_INVALID
    assert call(temp=float("inf")) == ttv.TTV_ERR_INVALID
    assert call(p=1.5) == ttv.TTV_ERR_INVALID
    assert call(p=-0.1) == ttv.TTV_ERR_INVALID
    assert call(ustride=-1) == ttv.TTV_ERR_INVALID
    assert call(u=None) == ttv.TTV_ERR_INVALID
    assert call(stride=100) == ttv.TTV_ERR_INVALID
    assert call(n_rows=70000) == ttv.TTV_ERR_INVALID
    assert call(wsb=need - 8) == ttv.TTV_ERR_WORKSPACE
    assert call(k=64, vocab=6000000, stride=6000000, wsb=1 << 40) == ttv.TTV_ERR_INVALID  # too many candidates
    assert "candidates" in ttv.last_error()
    assert call(n_rows=0) == ttv.TTV_OK


def test_walk_validation():
    b, keep = batch([0, 0], [5])
    f = C["tree_accept_walk"]
    assert f(ctypes.byref(b), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, None, FAKE, None) == ttv.TTV_ERR_INVALID
    b, keep = batch([0, 4], [5])
    assert f(ctypes.byref(b), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 8, None, FAKE, None) == ttv.TTV_ERR_INVALID
    assert "sel_stride" in ttv.last_error()


def test_can_gather_refusals():
    st, msg = ttv.kv_can_gather_raw([layer(dtype=ttv.TTV_I8)])
    assert st == ttv.TTV_ERR_UNSUPPORTED and "scale" in msg
    st, msg = ttv.kv_can_gather_raw([layer(), ttv.TtvKvLayer(None, FAKE, None, None, ttv.TTV_BF16, 8, 128, 64)])
    assert st == ttv.TTV_ERR_UNSUPPORTED and "layer 1" in msg
    st, msg = ttv.kv_can_gather_raw([layer(dtype=7)])
    assert st == ttv.TTV_ERR_UNSUPPORTED
    st, msg = ttv.kv_can_gather_raw([layer(dtype=ttv.TTV_I8, D=8, scales=True)])
    assert st == ttv.TTV_ERR_UNSUPPORTED
    assert ttv.kv_can_gather_raw([layer(dtype=ttv.TTV_I8, scales=True), layer(dtype=ttv.TTV_F32, D=64)])[0] == 0


def _gather(src, dst, B=2, live=(100, 100), ws=1 << 20, sel_stride=128):
    live = np.asarray(live, np.int32)
    return C["kv_gather_positions"]((ttv.TtvKvLayer * len(src))(*src),
                                    None if dst is None else (ttv.TtvKvLayer * len(dst))(*dst), len(src), B, FAKE,
                                    sel_stride, FAKE, live.ctypes.data, FAKE, FAKE, ws, None)


def test_gather_validation():
    base = 1 << 30
    mk = lambda off, cap=128: ttv.TtvKvLayer(base + off, base + off + (1 << 24), None, None, ttv.TTV_BF16, 2, 64, cap)
    # partial aliasing: dst starts inside src's K buffer
    assert _gather([mk(0)], [mk(4096)]) == ttv.TTV_ERR_INVALID
    assert "overlaps" in ttv.last_error()
    # live length beyond capacity
    assert _gather([mk(0)], None, live=(100, 200)) == ttv.TTV_ERR_INVALID
    # workspace too small
    assert _gather([mk(0)], None, ws=4) == ttv.TTV_ERR_WORKSPACE
    # shape mismatch between src and dst
    assert _gather([mk(0)], [mk(1 << 28, cap=256)]) == ttv.TTV_ERR_INVALID
    # int8 without sidecars: a named refusal
    i8 = ttv.TtvKvLayer(base, base + (1 << 24), None, None, ttv.TTV_I8, 2, 64, 128)
    assert _gather([i8], None) == ttv.TTV_ERR_UNSUPPORTED
    # j0 and bad per sequence, plus a partial pair per validation chunk (at most 64)
    assert ttv.kv_gather_positions_ws(8) == 8 * (2 + 2 * 64) * 4


def test_gather_refuses_rows_wider_than_one_pass():
    """Rows over 4096 bytes are refused by the capability question and by
    both gather entry points (in place and out of place) before anything is
    launched; 4096-byte rows are accepted."""
    base = 1 << 30
    wide = ttv.TtvKvLayer(base, base + (1 << 28), None, None, ttv.TTV_F32, 2, 1040, 128)   # 4160-byte rows
    edge = ttv.TtvKvLayer(base, base + (1 << 28), None, None, ttv.TTV_F32, 2, 1024, 128)   # 4096-byte rows
    st, msg = ttv.kv_can_gather_raw([wide])
    assert st == ttv.TTV_ERR_UNSUPPORTED and "4160-byte rows" in msg
    assert ttv.kv_can_gather_raw([edge])[0] == ttv.TTV_OK
    big8 = ttv.TtvKvLayer(base, base + (1 << 28), FAKE, FAKE, ttv.TTV_I8, 2, 4112, 128)
    assert ttv.kv_can_gather_raw([big8])[0] == ttv.TTV_ERR_UNSUPPORTED
    assert _gather([wide], None) == ttv.TTV_ERR_UNSUPPORTED                  # in place
    assert "wider than the gather moves" in ttv.last_error()
    dst = ttv.TtvKvLayer(base + (1 << 29), base + (1 << 29) + (1 << 28), None, None, ttv.TTV_F32, 2, 1040, 128)
    assert _gather([wide], [dst]) == ttv.TTV_ERR_UNSUPPORTED                 # out of place
    assert _tail([wide]) == ttv.TTV_ERR_UNSUPPORTED                          # tail form
    assert "wider than the gather moves" in ttv.last_error()


def test_sliding_mask_validation():
    f = C["sliding_mask_from_caller"]
    assert f(FAKE, 4, 10, 6, 0, -1e9, FAKE + (1 << 20), None) == ttv.TTV_ERR_INVALID   # window 0
    assert "window" in ttv.last_error()
    assert f(FAKE, -1, 10, 6, 4, -1e9, FAKE + (1 << 20), None) == ttv.TTV_ERR_INVALID
    assert f(FAKE, 4, 10, -6, 4, -1e9, FAKE + (1 << 20), None) == ttv.TTV_ERR_INVALID
    assert f(FAKE, 70000, 10, 6, 4, -1e9, FAKE + (1 << 24), None) == ttv.TTV_ERR_INVALID
    assert f(FAKE, 4, 10, 0x7FFFFFFF - 2, 4, -1e9, FAKE + (1 << 20), None) == ttv.TTV_ERR_INVALID
    assert f(None, 4, 10, 6, 4, -1e9, FAKE, None) == ttv.TTV_ERR_INVALID
    # out starting inside caller: partial overlap is refused, exact aliasing is not checked here
    assert f(FAKE, 4, 10, 6, 4, -1e9, FAKE + 8, None) == ttv.TTV_ERR_INVALID
    assert "overlap" in ttv.last_error()
    # empty shapes are a no-op
    assert f(None, 0, 10, 6, 4, -1e9, None, None) == ttv.TTV_OK
    assert f(None, 3, 0, 6, 4, -1e9, None, None) == ttv.TTV_OK


def _tail(layers, B=2, live=(100, 100), tail=(16, 16), wrapped=None, ws=1 << 20, stride=64):
    live = np.asarray(live, np.int32)
    tail = np.asarray(tail, np.int32)
    w = None if wrapped is None else np.asarray(wrapped, np.int32)
    return C["kv_gather_within_tail"]((ttv.TtvKvLayer * len(layers))(*layers), len(layers), B, FAKE, stride, FAKE,
                                      live.ctypes.data, tail.ctypes.data, None if w is None else w.ctypes.data, FAKE,
                                      FAKE, ws, None)


def test_tail_gather_validation_and_ring_refusal():
    L = [layer(cap=128)]
    # a wrapped rotating cache is refused by name before anything launches
    assert _tail(L, wrapped=(0, 1)) == ttv.TTV_ERR_UNSUPPORTED
    assert "sequence 1 has wrapped" in ttv.last_error()
    arr = (ttv.TtvKvLayer * 1)(*L)
    w = np.array([1, 0], np.int32)
    assert C["kv_can_gather_within_tail"](arr, 1, 2, w.ctypes.data) == ttv.TTV_ERR_UNSUPPORTED
    assert "sequence 0" in ttv.last_error()
    assert C["kv_can_gather_within_tail"](arr, 1, 2, None) == ttv.TTV_OK
    w[:] = 0
    assert C["kv_can_gather_within_tail"](arr, 1, 2, w.ctypes.data) == ttv.TTV_OK
    # the layer refusals of kv_can_gather carry over
    i8 = (ttv.TtvKvLayer * 1)(layer(dtype=ttv.TTV_I8))
    assert C["kv_can_gather_within_tail"](i8, 1, 2, None) == ttv.TTV_ERR_UNSUPPORTED
    # tail longer than the live window, than a tree block, or negative
    assert _tail(L, tail=(16, 101)) == ttv.TTV_ERR_INVALID
    assert _tail(L, live=(100, 120), tail=(16, 65)) == ttv.TTV_ERR_INVALID
    assert "tail_len[1]" in ttv.last_error()
    assert _tail(L, tail=(-1, 3)) == ttv.TTV_ERR_INVALID
    assert _tail(L, live=(100, 129)) == ttv.TTV_ERR_INVALID                   # beyond cap
    assert _tail(L, ws=4) == ttv.TTV_ERR_WORKSPACE
    assert _tail(L, stride=-1) == ttv.TTV_ERR_INVALID
    assert _tail([layer(cap=128), layer(cap=256)]) == ttv.TTV_ERR_INVALID     # layers differ
    assert ttv.kv_gather_within_tail_ws(8) == 8 * 4 * 4
    assert ttv.kv_gather_within_tail_ws(0) == 0


def test_window_attention_validation():
    b, keep = batch([0, 4], [10])
    L = layer()
    assert C["tree_verify_attention_window_ws"](ctypes.byref(b), 40, ctypes.byref(L), ttv.TTV_BF16, 0) == 0
    assert C["tree_verify_attention_window_ws"](ctypes.byref(b), 40, ctypes.byref(L), ttv.TTV_BF16, 64) > 0
    st = C["tree_verify_attention_window"](ctypes.byref(b), FAKE, ttv.TTV_BF16, 40, ctypes.byref(L), None, 0.1, 0,
                                           FAKE, FAKE, 1 << 30, None)
    assert st == ttv.TTV_ERR_INVALID and "window" in ttv.last_error()
    # a small workspace is refused before anything launches
    st = C["tree_verify_attention_window"](ctypes.byref(b), FAKE, ttv.TTV_BF16, 40, ctypes.byref(L), None, 0.1, 8,
                                           FAKE, FAKE, 4, None)
    assert st == ttv.TTV_ERR_WORKSPACE


def test_draft_validation():
    E, S = C["draft_tree_expand"], C["draft_tree_select"]
    V = 248320
    ws = C["draft_tree_expand_ws"](16, V, 4)
    nc = (V + 2047) // 2048  # 2,048-logit chunks: 4 candidates (8 B) and 16 B of statistics each
    assert ws == 16 * nc * 4 * 8 + 16 * nc * 16

    def expand(B=2, depth=1, k=4, vocab=V, stride=V, cap=128, ws_bytes=ws, logits=FAKE):
        return E(B, depth, k, logits, vocab, stride, FAKE, FAKE, FAKE, FAKE, cap, FAKE, FAKE, FAKE, ws_bytes, None)

    assert expand(B=0) == ttv.TTV_ERR_INVALID and "B 0" in ttv.last_error()
    assert expand(depth=0) == ttv.TTV_ERR_INVALID
    assert expand(k=17) == ttv.TTV_ERR_INVALID and "top_k 17" in ttv.last_error()
    assert expand(vocab=3) == ttv.TTV_ERR_INVALID
    assert expand(stride=V - 1) == ttv.TTV_ERR_INVALID and "row_stride" in ttv.last_error()
    assert expand(cap=4097) == ttv.TTV_ERR_INVALID and "cand_cap" in ttv.last_error()
    assert expand(cap=3) == ttv.TTV_ERR_INVALID
    assert expand(logits=None) == ttv.TTV_ERR_INVALID and "NULL" in ttv.last_error()
    assert expand(ws_bytes=ws - 1, B=16) == ttv.TTV_ERR_WORKSPACE
    # depth > 1 reads top_k rows per sequence: 4 sequences need the ws of 16 rows
    assert expand(B=4, depth=2, ws_bytes=ws - 1) == ttv.TTV_ERR_WORKSPACE
    assert expand(k=16, vocab=1 << 30, stride=1 << 30, ws_bytes=1 << 62) == ttv.TTV_ERR_INVALID

    def select(B=2, n=16, cap=128, out=FAKE):
        return S(B, n, FAKE, FAKE, FAKE, FAKE, FAKE, cap, out, FAKE, None, FAKE, None)

    assert select(n=65) == ttv.TTV_ERR_INVALID and "n_nodes 65" in ttv.last_error()
    assert select(n=0) == ttv.TTV_ERR_INVALID
    assert select(B=129) == ttv.TTV_ERR_INVALID
    assert select(cap=0) == ttv.TTV_ERR_INVALID
    assert select(out=None) == ttv.TTV_ERR_INVALID


def test_lm_head_validation():
    A = C["lm_head_argmax"]
    V, H = 248320, 5120
    ws = C["lm_head_argmax_ws"](16, V)
    assert ws == 16 * ((V + 511) // 512) * 8
    # up to 112 nodes a workgroup covers 512 vocabulary rows, beyond that 256
    assert C["lm_head_argmax_ws"](112, V) == 112 * ((V + 511) // 512) * 8
    assert C["lm_head_argmax_ws"](113, V) == 113 * ((V + 255) // 256) * 8
    assert C["lm_head_argmax_ws"](300, V) == 300 * ((V + 255) // 256) * 8

    def call(n=16, hs=H, w=FAKE, v=V, h=H, wst=H, out=FAKE, ws_bytes=ws, x=FAKE):
        return A(x, n, hs, w, v, h, wst, out, FAKE, ws_bytes, None)

    assert call(n=0) == ttv.TTV_OK  # nothing to do
    assert call(n=-1) == ttv.TTV_ERR_INVALID
    assert call(v=0) == ttv.TTV_ERR_INVALID and "vocab" in ttv.last_error()
    assert call(h=100, hs=104, wst=104) == ttv.TTV_ERR_INVALID and "multiple of 64" in ttv.last_error()
    assert call(hs=H - 8) == ttv.TTV_ERR_INVALID and "strides" in ttv.last_error()
    assert call(wst=H + 4) == ttv.TTV_ERR_INVALID
    assert call(w=None) == ttv.TTV_ERR_INVALID and "NULL" in ttv.last_error()
    assert call(x=FAKE + 2) == ttv.TTV_ERR_INVALID and "aligned" in ttv.last_error()
    assert call(ws_bytes=ws - 1) == ttv.TTV_ERR_WORKSPACE


def test_lm_head_q4_validation():
    A = C["lm_head_q4_argmax"]
    V, H = 248320, 5120
    ws = C["lm_head_q4_argmax_ws"](16, V, H)
    # best keys per (node, 256-row slab), 256-byte aligned, then the group
    # sums as three bf16 planes of 16 nodes x (groups rounded up to 32)
    assert ws == (16 * ((V + 255) // 256) * 8 + 255) // 256 * 256 + 3 * 16 * 96 * 2
    assert C["lm_head_q4_argmax_ws"](16, V, 32) == 0

    def call(n=16, hs=H, v=V, h=H, wq=FAKE, sb=FAKE, x=FAKE, ws_bytes=ws):
        return A(x, n, hs, wq, sb, v, h, FAKE, FAKE, ws_bytes, None)

    assert call(n=0) == ttv.TTV_OK
    assert call(v=V + 2) == ttv.TTV_ERR_INVALID and "multiple of 4" in ttv.last_error()
    assert call(h=96, hs=96) == ttv.TTV_ERR_INVALID and "multiple of 64" in ttv.last_error()
    assert call(hs=H + 4) == ttv.TTV_ERR_INVALID
    assert call(sb=None) == ttv.TTV_ERR_INVALID and "NULL" in ttv.last_error()
    assert call(sb=FAKE + 8) == ttv.TTV_ERR_INVALID and "aligned" in ttv.last_error()
    assert call(wq=FAKE + 4) == ttv.TTV_ERR_INVALID
    assert call(ws_bytes=ws - 1) == ttv.TTV_ERR_WORKSPACE
