"""The allocation-free attention entry point (tree_verify_attention_static):
its output must equal tree_verify_attention's on the same inputs, call after
call, with the static scratch reused by a smaller call after a larger one."""

import math

import numpy as np
import pytest
import torch

import oracle as O
from workloads import config2_round, config3_round, config5_round, host_tensors

from gpu_util import layer_to_dev, log, run_attention, run_mask, spec_batch, to_dev, to_host, zeros_ws

pytestmark = pytest.mark.gpu

TOL_BF16 = 2e-3


@pytest.fixture(scope="module")
def ttv():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from gpu_util import binding
    return binding()


def _static_vs_workspace(ttv, batch, q, layer, anc, scale):
    ws_out, _ = run_attention(ttv, batch, q, layer, anc, scale, ws=zeros_ws(
        ttv.tree_verify_attention_ws(batch, q.shape[1], layer, "bf16")).fill_(0xA5))
    st_out = torch.full_like(ws_out, float("nan"))
    ttv.tree_verify_attention_static(batch, q, layer, anc, scale, st_out)
    torch.cuda.synchronize()
    return ws_out, st_out


def test_static_scratch_matches_workspace_entry_point(ttv):
    # 1. the long-context layer at full size (B=8, 131,072-token prefix, int8 KV), the largest call
    from workloads.device import dev_kv_cache, dev_queries
    spec = config5_round(0, [131072] * 8, "tree", L=1)
    cap = int(max(spec.hist_len + np.diff(spec.node_off)))
    c = dev_kv_cache(spec.seed, 100, spec.B, spec.Hkv, cap, spec.D, "i8", "cuda")
    layer = ttv.KVLayer(c["k"], c["v"], c["k_scale"], c["v_scale"])
    need = ttv.tree_verify_attention_ws(spec_batch(ttv, spec), spec.Hq, layer, "bf16")
    assert 0 < need <= ttv.STATIC_SCRATCH_BYTES
    q = dev_queries(spec.seed, 200, spec.n_nodes, spec.Hq, spec.D, "bf16", "cuda")
    batch = spec_batch(ttv, spec)
    anc, _, st = run_mask(ttv, batch, to_dev(spec.flat("parents")))
    a, b = _static_vs_workspace(ttv, batch, q, layer, anc, 1 / math.sqrt(spec.D))
    log(f"static scratch, long-context layer ({need} bytes of partials): equal {torch.equal(a, b)}")
    assert torch.equal(a, b)
    assert bool(torch.isfinite(b).all())
    del c, layer
    # 2. then smaller calls on the same scratch: a 16-node int8 tree over 6,000 keys, then a bf16 chain
    prev = need
    for spec in (config3_round(P=6000, L=1), config2_round(8, 3)):
        tens = host_tensors(spec)
        host = tens["layers"][0]
        dev, kvl = layer_to_dev(ttv, host)
        batch = spec_batch(ttv, spec)
        need = ttv.tree_verify_attention_ws(batch, spec.Hq, kvl, "bf16")
        assert 0 < need < prev
        prev = need
        anc, _, st = run_mask(ttv, batch, to_dev(spec.flat("parents")))
        q = to_dev(host["q"], "bf16")
        a, b = _static_vs_workspace(ttv, batch, q, kvl, anc, 1 / math.sqrt(spec.D))
        assert int(st.item()) == 0
        assert torch.equal(a, b), spec.note
        want = O.tree_verify_attention(host["q"], {k: v for k, v in host.items() if k != "q"}, spec.node_off,
                                       spec.hist_len, spec.parents, 1 / math.sqrt(spec.D), "bf16", spec.kv_dtype)
        err = float(np.abs(to_host(b) - want).max())
        log(f"static scratch, {spec.note or spec.kv_dtype} ({need} bytes): equal, max|err| vs oracle {err:.2e}")
        assert err <= TOL_BF16


def test_static_scratch_refuses_calls_beyond_its_size(ttv):
    """A call whose partials exceed the static scratch is refused on the host
    with TTV_ERR_UNSUPPORTED and writes nothing."""
    from workloads import config4_round
    spec = config4_round()
    cap = int(max(spec.hist_len + np.diff(spec.node_off)))
    import ctypes
    k = torch.zeros(1, 1, dtype=torch.bfloat16, device="cuda")
    batch = spec_batch(ttv, spec)
    L = ttv.TtvKvLayer(k.data_ptr(), k.data_ptr(), None, None, ttv.TTV_BF16, spec.Hkv, spec.D, cap)
    assert ttv._c["tree_verify_attention_ws"](batch.ref(), spec.Hq, ctypes.byref(L), ttv.TTV_BF16) > \
        ttv.STATIC_SCRATCH_BYTES
    out = torch.full((spec.n_nodes, spec.Hq, spec.D), 7.0, device="cuda")
    st = ttv._c["tree_verify_attention_static"](batch.ref(), k.data_ptr(), ttv.TTV_BF16, spec.Hq, ctypes.byref(L),
                                                None, 0.1, out.data_ptr(), None)
    assert st == ttv.TTV_ERR_UNSUPPORTED and "static scratch" in ttv.last_error()
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
