"""Race check: every kernel computes each work item (a query or key tile of
one head, a key range of one sequence) in one workgroup, with no atomics and
no communication between workgroups, so its results cannot depend on the
order in which the workgroups run. The library's debug switch reverses that
order; each path below runs both ways on the same inputs and must give
bitwise identical outputs. A difference would expose a race such as an LDS
buffer refilled before every wave finished reading it.
"""
import numpy as np
import pytest
import torch

import io_aware_exact_10_amd as fa
import synth
from gpu_util import announce, to_device

pytestmark = pytest.mark.gpu

NONE, CAUSAL, BSP = synth.MASK_NONE, synth.MASK_CAUSAL, synth.MASK_BLOCK_SPARSE


def both_orders(fn):
    """fn() -> tuple of tensors, run in the usual and the reversed order."""
    prev = fa.fa_debug_reverse_order(0)
    try:
        a = [x.clone() for x in fn()]
        torch.cuda.synchronize()
        fa.fa_debug_reverse_order(1)
        b = [x.clone() for x in fn()]
        torch.cuda.synchronize()
    finally:
        fa.fa_debug_reverse_order(prev)
    return a, b


def assert_same(a, b, what):
    for i, (x, y) in enumerate(zip(a, b)):
        assert torch.equal(x, y), f"{what}: output {i}"


@pytest.mark.parametrize("dtype", [synth.DTYPE_BF16, synth.DTYPE_F32])
@pytest.mark.parametrize("mask_kind", [NONE, CAUSAL, BSP])
@pytest.mark.parametrize("d", [64, 128])
def test_dense_fwd_bwd_order_independent(d, mask_kind, dtype):
    N = 1000 if dtype == synth.DTYPE_BF16 else 300
    w = synth.small_workload(2, 3, N, d, dtype, mask_kind, seed=9100 + d + mask_kind)
    t = to_device(synth.make_inputs(w))
    announce(f"reverse order: fa_fwd + fa_bwd N{N} d{d} mask{mask_kind} dtype{dtype}")

    def run():
        o, lse = fa.forward(t["q"], t["k"], t["v"], w.scale, mask_kind, t["mask"])
        return (o, lse) + tuple(fa.backward(t["q"], t["k"], t["v"], o, lse, t["do"], w.scale, mask_kind, t["mask"]))

    a, b = both_orders(run)
    assert_same(a, b, "dense")


@pytest.mark.parametrize("mask_kind", [NONE, CAUSAL])
@pytest.mark.parametrize("d", [64, 128])
def test_long_shape_order_independent(d, mask_kind):
    """The 256-row (eight-wave) forward shape."""
    w = synth.small_workload(1, 2, 2304, d, synth.DTYPE_BF16, mask_kind, seed=9200 + d + mask_kind)
    t = to_device(synth.make_inputs(w))
    announce(f"reverse order: fa_fwd_tiled 256 rows N{w.N} d{d} mask{mask_kind}")
    a, b = both_orders(lambda: fa.forward(t["q"], t["k"], t["v"], w.scale, mask_kind, None, block_rows=256))
    assert_same(a, b, "256-row forward")


@pytest.mark.parametrize("mask_kind", [NONE, CAUSAL])
def test_varlen_gqa_order_independent(mask_kind):
    lens = [130, 1, 700, 64, 333]
    p = synth.packed_inputs(lens, lens, 8, 2, 128, seed=9300 + mask_kind)
    dev = lambda bits: torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()
    q, k, v, do = dev(p.q_bits), dev(p.k_bits), dev(p.v_bits), dev(p.do_bits)
    cu = torch.from_numpy(p.cu_q).cuda()
    mx = max(lens)
    announce(f"reverse order: fa_fwd_varlen + fa_bwd_varlen lens{lens} mask{mask_kind}")

    def run():
        o, lse = fa.forward_varlen(q, k, v, cu, cu, mx, mx, p.scale, mask_kind)
        return (o, lse) + tuple(fa.backward_varlen(q, k, v, o, lse, do, cu, cu, mx, mx, p.scale, mask_kind))

    a, b = both_orders(run)
    assert_same(a, b, "varlen")


def test_splitkv_order_independent():
    qlens, klens = [1, 1, 2, 1], [3000, 17, 1024, 2049]
    p = synth.packed_inputs(qlens, klens, 8, 2, 128, seed=9400)
    dev = lambda bits: torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()
    q, k, v = dev(p.q_bits), dev(p.k_bits), dev(p.v_bits)
    cq, ck = torch.from_numpy(p.cu_q).cuda(), torch.from_numpy(p.cu_k).cuda()
    announce("reverse order: fa_fwd_splitkv")
    a, b = both_orders(lambda: fa.forward_splitkv(q, k, v, cq, ck, max(qlens), max(klens), p.scale, CAUSAL))
    assert_same(a, b, "split-key")


@pytest.mark.parametrize("mask_kind", [NONE, CAUSAL])
def test_fp8_order_independent(mask_kind):
    f = synth.fp8_inputs(2, 2, 700, 128, seed=9500 + mask_kind)
    t = [torch.from_numpy(np.ascontiguousarray(x)).cuda() for x in (f.q8, f.k8, f.vt8)]
    announce(f"reverse order: fa_fwd_fp8 mask{mask_kind}")
    a, b = both_orders(lambda: fa.forward_fp8(*t, f.q_descale, f.k_descale, f.v_descale, None, mask_kind))
    assert_same(a, b, "fp8")
