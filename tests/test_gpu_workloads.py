"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times: the whole batch runs on the GPU through the C ABI, and the
oracle recomputes sampled heads (all rows, or sampled rows for the 32K
prefill) one by one for comparison.
"""
import numpy as np
import pytest
import torch

import io_aware_exact_10_amd as fa
import oracle
import synth
from gpu_util import announce, check_forward, check_grad, to_device

pytestmark = pytest.mark.gpu


def sampled_heads(w):
    return sorted({(0, 0), (w.B - 1, w.H - 1), (w.B // 2, (w.H * 2) // 3)})


@pytest.mark.parametrize("name", ["gpt2_medium", "causal_train", "long_prefill", "block_sparse"])
def test_workload_sampled_heads(name):
    w = synth.WORKLOADS[name]
    inp = synth.make_inputs(w)
    t = to_device(inp)
    announce(f"fa_fwd full workload {name} B{w.B} H{w.H} N{w.N} d{w.d} mask{w.mask_kind}")
    o, lse = fa.forward(t["q"], t["k"], t["v"], w.scale, w.mask_kind, t["mask"])
    if w.backward:
        announce(f"fa_bwd full workload {name}")
        dq, dk, dv = fa.backward(t["q"], t["k"], t["v"], o, lse, t["do"], w.scale, w.mask_kind, t["mask"])
    torch.cuda.synchronize()
    assert torch.isfinite(lse).all() and torch.isfinite(o.float()).all()
    rows = None
    if w.N > 8192:
        rng = np.random.default_rng(w.seed)
        rows = np.unique(np.concatenate([np.arange(256), np.arange(w.N - 256, w.N),
                                         rng.choice(w.N, 256, replace=False)]))
    for b, h in sampled_heads(w):
        O, L = oracle.forward_head(inp.q[b, h], inp.k[b, h], inp.v[b, h], w.scale, w.mask_kind, inp.mask, rows)
        go = o[b, h].float().cpu().numpy()
        gl = lse[b, h].cpu().numpy()
        if rows is not None:
            go, gl = go[rows], gl[rows]
        check_forward(go, gl, O, L, w.dtype, f"{name} head ({b},{h})")
        if w.backward:
            gq, gk, gv = oracle.backward_head(inp.q[b, h], inp.k[b, h], inp.v[b, h], inp.do[b, h],
                                              w.scale, w.mask_kind, inp.mask)
            for n, got, ref in (("dq", dq, gq), ("dk", dk, gk), ("dv", dv, gv)):
                check_grad(got[b, h].float().cpu().numpy(), ref, w.dtype, f"{name} head ({b},{h}) {n}")
