"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times: the whole batch runs on the GPU through the C ABI, and the
oracle recomputes sampled heads (all rows), or for the 32K prefill every
head on sampled rows, one by one for comparison.
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
    heads = sampled_heads(w)
    if w.N > 8192:
        # long sequences: every head, on every 64th query row plus the first
        # and the last 64 rows (the shortest and the longest causal rows)
        rows = np.unique(np.concatenate([np.arange(0, w.N, 64), np.arange(64), np.arange(w.N - 64, w.N)]))
        heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    for b, h in heads:
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


def test_packed_workload_sampled_sequences():
    """The packed grouped-query workload at full size (16 causal sequences of
    up to 4096 tokens, 32 query heads over 8 K/V heads, d = 128): forward and
    backward of the whole batch on the GPU; the oracle recomputes sampled
    sequences, and for dK/dV every query head of one K/V group."""
    w = synth.PACKED_WORKLOADS["varlen_gqa"]
    lens = w.lengths()
    p = synth.packed_inputs(lens, lens, w.H, w.Hkv, w.d, w.seed)
    dev = lambda bits: torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()
    q, k, v, do = dev(p.q_bits), dev(p.k_bits), dev(p.v_bits), dev(p.do_bits)
    cu = torch.from_numpy(p.cu_q).cuda()
    mx = max(lens)
    announce(f"fa_fwd_varlen full workload {w.name} tokens {q.shape[0]} H{w.H}/{w.Hkv} d{w.d}")
    o, lse = fa.forward_varlen(q, k, v, cu, cu, mx, mx, w.scale, w.mask_kind)
    announce(f"fa_bwd_varlen full workload {w.name}")
    dq, dk, dv = fa.backward_varlen(q, k, v, o, lse, do, cu, cu, mx, mx, w.scale, w.mask_kind)
    torch.cuda.synchronize()
    assert torch.isfinite(lse).all() and torch.isfinite(o.float()).all()
    G = w.H // w.Hkv
    hk = 1
    for b in (6, int(np.argmax(lens))):
        a, e = int(p.cu_q[b]), int(p.cu_q[b + 1])
        ref_dk = np.zeros((e - a, w.d))
        ref_dv = np.zeros((e - a, w.d))
        for h in range(hk * G, (hk + 1) * G):
            args = (p.q[a:e, h], p.k[a:e, hk], p.v[a:e, hk])
            O, L = oracle.forward_head(*args, w.scale, w.mask_kind)
            check_forward(o[a:e, h].float().cpu().numpy(), lse[h, a:e].cpu().numpy(), O, L, synth.DTYPE_BF16,
                          f"{w.name} seq {b} head {h}")
            gq, gk, gv = oracle.backward_head(*args, p.do[a:e, h], w.scale, w.mask_kind)
            check_grad(dq[a:e, h].float().cpu().numpy(), gq, synth.DTYPE_BF16, f"{w.name} seq {b} head {h} dq")
            ref_dk += gk
            ref_dv += gv
        check_grad(dk[a:e, hk].float().cpu().numpy(), ref_dk, synth.DTYPE_BF16, f"{w.name} seq {b} kv head {hk} dk")
        check_grad(dv[a:e, hk].float().cpu().numpy(), ref_dv, synth.DTYPE_BF16, f"{w.name} seq {b} kv head {hk} dv")


def test_decode_workload_sampled_sequences():
    """The decoding workload at full size (one query per sequence against 64
    cached sequences of 1024..8192 keys, 32 query heads over 8 K/V heads,
    d = 128) through the split-key forward; the oracle recomputes every head
    of sampled sequences."""
    w = synth.PACKED_WORKLOADS["decode_splitkv"]
    lens, qlens = w.lengths(), w.query_lengths()
    p = synth.packed_inputs(qlens, lens, w.H, w.Hkv, w.d, w.seed)
    dev = lambda bits: torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()
    q, k, v = dev(p.q_bits), dev(p.k_bits), dev(p.v_bits)
    cq, ck = torch.from_numpy(p.cu_q).cuda(), torch.from_numpy(p.cu_k).cuda()
    announce(f"fa_fwd_splitkv full workload {w.name} keys {k.shape[0]} H{w.H}/{w.Hkv} d{w.d}")
    o, lse = fa.forward_splitkv(q, k, v, cq, ck, max(qlens), max(lens), w.scale, w.mask_kind)
    torch.cuda.synchronize()
    assert torch.isfinite(lse).all() and torch.isfinite(o.float()).all()
    G = w.H // w.Hkv
    for b in (0, int(np.argmax(lens)), int(np.argmin(lens)), w.B - 1):
        a, e = int(p.cu_q[b]), int(p.cu_q[b + 1])
        ka, ke = int(p.cu_k[b]), int(p.cu_k[b + 1])
        for h in range(w.H):
            O, L = oracle.forward_head(p.q[a:e, h], p.k[ka:ke, h // G], p.v[ka:ke, h // G], w.scale, w.mask_kind)
            check_forward(o[a:e, h].float().cpu().numpy(), lse[h, a:e].cpu().numpy(), O, L, synth.DTYPE_BF16,
                          f"{w.name} seq {b} head {h}")
