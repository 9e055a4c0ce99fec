"""GPU parity of the packed variable-length path (unequal query/key lengths
with the causal offset, shared K/V heads) through the C ABI against the CPU
float64 oracle on identical seeded inputs. Tolerances: tests/gpu_util.py.
"""
import numpy as np
import pytest
import torch

import io_aware_exact_10_amd as fa
import oracle
import synth
from gpu_util import announce, check_forward, check_grad, max_abs

pytestmark = pytest.mark.gpu

BF = synth.DTYPE_BF16
NONE, CAUSAL = synth.MASK_NONE, synth.MASK_CAUSAL


def dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def to_dev(p):
    return dict(q=dev(p.q_bits), k=dev(p.k_bits), v=dev(p.v_bits), do=dev(p.do_bits),
                cu_q=torch.from_numpy(p.cu_q).cuda(), cu_k=torch.from_numpy(p.cu_k).cuda())


def run_varlen(p, mask_kind, backward=True, scale=None, max_q=None, max_k=None, fill=None):
    """Forward (+ backward) through fa_fwd_varlen / fa_bwd_varlen. ``fill``
    pre-fills the outputs so that untouched rows can be checked."""
    scale = p.scale if scale is None else scale
    t = to_dev(p)
    mq = max(max(p.lens_q), 1) if max_q is None else max_q
    mk = max(max(p.lens_k), 1) if max_k is None else max_k
    o = lse = None
    if fill is not None:
        o = torch.full_like(t["q"], fill)
        lse = torch.full((p.H, p.q.shape[0]), fill, dtype=torch.float32, device="cuda")
    announce(f"fa_fwd_varlen {p.name} lens_q{p.lens_q} lens_k{p.lens_k} mask{mask_kind} seed{p.seed}")
    o, lse = fa.forward_varlen(t["q"], t["k"], t["v"], t["cu_q"], t["cu_k"], mq, mk, scale, mask_kind,
                               out=o, lse=lse)
    torch.cuda.synchronize()
    out = dict(o=o.float().cpu().numpy().astype(np.float64), lse=lse.cpu().numpy().astype(np.float64))
    if backward:
        announce(f"fa_bwd_varlen {p.name}")
        grads = None
        if fill is not None:
            grads = dict(dq=torch.full_like(t["q"], fill), dk=torch.full_like(t["k"], fill),
                         dv=torch.full_like(t["v"], fill))
        else:
            grads = {}
        dq, dk, dv = fa.backward_varlen(t["q"], t["k"], t["v"], o, lse, t["do"], t["cu_q"], t["cu_k"], mq, mk,
                                        scale, mask_kind, **grads)
        torch.cuda.synchronize()
        for n, x in (("dq", dq), ("dk", dk), ("dv", dv)):
            out[n] = x.float().cpu().numpy().astype(np.float64)
    return out


def oracle_varlen(p, mask_kind, backward=True, scale=None):
    scale = p.scale if scale is None else scale
    O, L = oracle.forward_varlen(p.q, p.k, p.v, p.cu_q, p.cu_k, scale, mask_kind)
    ref = dict(o=O, lse=L)
    if backward:
        ref["dq"], ref["dk"], ref["dv"] = oracle.backward_varlen(p.q, p.k, p.v, p.do, p.cu_q, p.cu_k, scale,
                                                                 mask_kind)
    return ref


def compare_covered(p, got, ref, backward=True):
    """Compare the rows that belong to a sequence."""
    tq, tk = int(p.cu_q[-1]), int(p.cu_k[-1])
    check_forward(got["o"][:tq], got["lse"][:, :tq], ref["o"][:tq], ref["lse"][:, :tq], BF, p.name)
    if backward:
        check_grad(got["dq"][:tq], ref["dq"][:tq], BF, f"{p.name} dq")
        check_grad(got["dk"][:tk], ref["dk"][:tk], BF, f"{p.name} dk")
        check_grad(got["dv"][:tk], ref["dv"][:tk], BF, f"{p.name} dv")


CASES = [
    # (lens_q, lens_k): ragged lengths across tile edges, an empty sequence,
    # a one-token query, more keys than queries and (causal) more queries
    # than keys, whose first rows then see no key.
    ([1, 130, 257, 64, 0, 300], [1, 200, 257, 100, 37, 129]),
    ([65, 1, 333], [65, 513, 200]),
]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("H,Hkv", [(4, 4), (8, 2), (6, 1)])
@pytest.mark.parametrize("mask_kind", [NONE, CAUSAL])
@pytest.mark.parametrize("case", [0, 1])
def test_varlen_gqa_parity(case, mask_kind, H, Hkv, d):
    lq, lk = CASES[case]
    p = synth.packed_inputs(lq, lk, H, Hkv, d, seed=5000 + 10 * case + H + Hkv + d + mask_kind)
    got = run_varlen(p, mask_kind)
    compare_covered(p, got, oracle_varlen(p, mask_kind))


@pytest.mark.parametrize("mask_kind", [NONE, CAUSAL])
def test_unequal_lengths_single_sequence(mask_kind):
    """One sequence, 200 queries against 1000 keys (a chunk appended to a
    cached prefix), d = 128, and the transposed case (1000 queries, 200 keys)."""
    for lq, lk in (([200], [1000]), ([1000], [200])):
        p = synth.packed_inputs(lq, lk, 4, 2, 128, seed=5100 + lq[0] + mask_kind)
        got = run_varlen(p, mask_kind)
        ref = oracle_varlen(p, mask_kind)
        compare_covered(p, got, ref)
        if mask_kind == CAUSAL and lq[0] > lk[0]:
            e = lq[0] - lk[0]
            assert (got["o"][:e] == 0).all() and np.isneginf(got["lse"][:, :e]).all()
            assert (got["dq"][:e] == 0).all()


def test_decode_shaped_queries():
    """One query per sequence against long, ragged key sequences."""
    p = synth.packed_inputs([1, 1, 1, 1], [1000, 37, 513, 64], 8, 1, 128, seed=5200)
    for mk in (NONE, CAUSAL):
        got = run_varlen(p, mk)
        compare_covered(p, got, oracle_varlen(p, mk))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("mask_kind", [NONE, CAUSAL])
def test_packed_equal_lengths_bitwise_equals_dense(mask_kind, d):
    """Equal lengths and Hkv = H: the packed call runs the same arithmetic as
    fa_fwd / fa_bwd on the [B, H, N, d] transpose, so results are bitwise equal.
    Under a causal mask the dense call gives each workgroup a pair of tiles
    (j, n - 1 - j) and the packed call one tile, so this also checks the two
    schedules against each other (N = 333: three tiles, one without a partner)."""
    B, H, N = 3, 4, 333
    p = synth.packed_inputs([N] * B, [N] * B, H, H, d, seed=5300 + d + mask_kind)
    got = run_varlen(p, mask_kind)
    t = to_dev(p)
    dense = lambda x: x.view(B, N, H, d).permute(0, 2, 1, 3).contiguous()
    announce(f"dense twin B{B} H{H} N{N} d{d} mask{mask_kind}")
    q, k, v, do = (dense(t[n]) for n in ("q", "k", "v", "do"))
    o, lse = fa.forward(q, k, v, None, mask_kind)
    dq, dk, dv = fa.backward(q, k, v, o, lse, do, None, mask_kind)
    torch.cuda.synchronize()
    back = lambda x: x.permute(0, 2, 1, 3).reshape(B * N, H, d).float().cpu().numpy()
    assert np.array_equal(got["o"], back(o))
    assert np.array_equal(got["lse"], lse.permute(1, 0, 2).reshape(H, B * N).cpu().numpy())
    for n, x in (("dq", dq), ("dk", dk), ("dv", dv)):
        assert np.array_equal(got[n], back(x)), n


# Random dense shapes (seeded): B, H in 1..4, N in 1..700, d in {64, 128}.
_PAIR_SHAPES = [(int(b), int(h), int(n), int(d)) for b, h, n, d in zip(
    np.random.default_rng(71).integers(1, 5, 12), np.random.default_rng(72).integers(1, 5, 12),
    np.random.default_rng(73).integers(1, 701, 12), np.random.default_rng(74).choice([64, 128], 12))]


@pytest.mark.parametrize("B,H,N,d", _PAIR_SHAPES)
def test_causal_pairs_bitwise_equal_single_tiles(B, H, N, d):
    """Causal work pairs (dense call: a workgroup takes query or key tiles j
    and n - 1 - j) against one tile per workgroup (packed call of the same
    equal-length sequences): the per-tile arithmetic is the same, so O, LSE
    and all gradients must agree bit for bit at any tile count, odd or even."""
    p = synth.packed_inputs([N] * B, [N] * B, H, H, d, seed=7100 + N)
    got = run_varlen(p, CAUSAL)
    t = to_dev(p)
    dense = lambda x: x.view(B, N, H, d).permute(0, 2, 1, 3).contiguous()
    announce(f"dense pairs B{B} H{H} N{N} d{d}")
    q, k, v, do = (dense(t[n]) for n in ("q", "k", "v", "do"))
    o, lse = fa.forward(q, k, v, None, CAUSAL)
    dq, dk, dv = fa.backward(q, k, v, o, lse, do, None, CAUSAL)
    torch.cuda.synchronize()
    back = lambda x: x.permute(0, 2, 1, 3).reshape(B * N, H, d).float().cpu().numpy()
    assert np.array_equal(got["o"], back(o))
    assert np.array_equal(got["lse"], lse.permute(1, 0, 2).reshape(H, B * N).cpu().numpy())
    for n, x in (("dq", dq), ("dk", dk), ("dv", dv)):
        assert np.array_equal(got[n], back(x)), n


def test_rows_outside_every_sequence_are_untouched():
    """Tokens past the last offset keep what the caller stored there."""
    p = synth.packed_inputs([70, 0, 150], [90, 33, 150], 4, 2, 64, seed=5400, pad_q=37, pad_k=21)
    got = run_varlen(p, CAUSAL, fill=7.0)
    tq, tk = int(p.cu_q[-1]), int(p.cu_k[-1])
    assert (got["o"][tq:] == 7.0).all() and (got["lse"][:, tq:] == 7.0).all()
    assert (got["dq"][tq:] == 7.0).all()
    assert (got["dk"][tk:] == 7.0).all() and (got["dv"][tk:] == 7.0).all()
    # key tokens of the sequence without queries: zero gradient
    ks = slice(int(p.cu_k[1]), int(p.cu_k[2]))
    assert (got["dk"][ks] == 0).all() and (got["dv"][ks] == 0).all()
    compare_covered(p, got, oracle_varlen(p, CAUSAL))


def test_max_seqlen_larger_than_needed():
    """A generous max_seqlen only adds workgroups that exit at once."""
    p = synth.packed_inputs([100, 17], [120, 17], 4, 4, 64, seed=5500)
    a = run_varlen(p, CAUSAL)
    b = run_varlen(p, CAUSAL, max_q=1000, max_k=2000)
    for n in a:
        assert max_abs(a[n], b[n]) == 0.0, n


@pytest.mark.parametrize("scale", [-0.3, 0.0])
def test_varlen_scale_sign_and_zero(scale):
    p = synth.packed_inputs([40, 200], [90, 200], 4, 2, 128, seed=5600)
    got = run_varlen(p, CAUSAL, scale=scale)
    compare_covered(p, got, oracle_varlen(p, CAUSAL, scale=scale))
