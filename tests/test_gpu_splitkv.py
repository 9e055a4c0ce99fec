"""GPU parity of the split-key forward (fa_fwd_splitkv: few queries per
sequence, long keys, key ranges merged by the block-combine rule) through the
C ABI against the CPU float64 oracle. Tolerances: tests/gpu_util.py.
"""
import numpy as np
import pytest
import torch

import io_aware_exact_10_amd as fa
import oracle
import synth
from gpu_util import announce, check_forward

pytestmark = pytest.mark.gpu

BF = synth.DTYPE_BF16
NONE, CAUSAL = synth.MASK_NONE, synth.MASK_CAUSAL


def dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def run_splitkv(p, mask_kind, num_splits=0, scale=None, fill=None):
    scale = p.scale if scale is None else scale
    q, k, v = dev(p.q_bits), dev(p.k_bits), dev(p.v_bits)
    cq, ck = torch.from_numpy(p.cu_q).cuda(), torch.from_numpy(p.cu_k).cuda()
    mq, mk = max(max(p.lens_q), 1), max(max(p.lens_k), 1)
    o = lse = None
    if fill is not None:
        o = torch.full_like(q, fill)
        lse = torch.full((p.H, q.shape[0]), fill, dtype=torch.float32, device="cuda")
    announce(f"fa_fwd_splitkv {p.name} lens_q{p.lens_q} lens_k{p.lens_k} mask{mask_kind} splits{num_splits} "
             f"seed{p.seed}")
    o, lse = fa.forward_splitkv(q, k, v, cq, ck, mq, mk, scale, mask_kind, num_splits, out=o, lse=lse)
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def check(p, mask_kind, got, scale=None):
    scale = p.scale if scale is None else scale
    O, L = oracle.forward_varlen(p.q, p.k, p.v, p.cu_q, p.cu_k, scale, mask_kind)
    tq = int(p.cu_q[-1])
    check_forward(got[0][:tq], got[1][:, :tq], O[:tq], L[:, :tq], BF, p.name)


CASES = [
    # decode: one query per sequence; ragged key lengths across tile edges
    ([1, 1, 1, 1, 1], [1000, 37, 4097, 1, 64]),
    # a few new tokens per sequence (speculative / chunked decoding)
    ([4, 16, 1, 7], [4096, 300, 2049, 7]),
]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("H,Hkv", [(32, 8), (8, 1), (4, 4)])
@pytest.mark.parametrize("mask_kind", [NONE, CAUSAL])
@pytest.mark.parametrize("case", [0, 1])
def test_splitkv_parity(case, mask_kind, H, Hkv, d):
    lq, lk = CASES[case]
    p = synth.packed_inputs(lq, lk, H, Hkv, d, seed=7000 + 10 * case + H + Hkv + d + mask_kind)
    check(p, mask_kind, run_splitkv(p, mask_kind))


@pytest.mark.parametrize("num_splits", [1, 2, 3, 17, 128])
def test_splitkv_forced_split_counts(num_splits):
    """Any number of key ranges, including more ranges than key tiles (empty
    ranges), gives the same attention."""
    p = synth.packed_inputs([1, 3, 2], [777, 2000, 65], 16, 4, 128, seed=7100)
    for mk in (NONE, CAUSAL):
        check(p, mk, run_splitkv(p, mk, num_splits))


def test_splitkv_matches_varlen_forward():
    """Same inputs through fa_fwd_varlen and fa_fwd_splitkv: both within the
    bf16 tolerance of each other (they round differently)."""
    p = synth.packed_inputs([2, 1, 5], [3000, 129, 640], 8, 2, 128, seed=7200)
    a = run_splitkv(p, CAUSAL)
    q, k, v = dev(p.q_bits), dev(p.k_bits), dev(p.v_bits)
    cq, ck = torch.from_numpy(p.cu_q).cuda(), torch.from_numpy(p.cu_k).cuda()
    announce("fa_fwd_varlen twin of the split-key case")
    o, lse = fa.forward_varlen(q, k, v, cq, ck, 5, 3000, None, CAUSAL)
    torch.cuda.synchronize()
    check_forward(a[0], a[1], o.float().cpu().numpy(), lse.cpu().numpy(), BF, "splitkv vs varlen")


def test_splitkv_empty_rows_and_untouched_tokens():
    """More queries than keys (causal): the first rows see nothing (O = 0,
    LSE = -inf); a sequence without keys likewise; tokens outside every
    sequence keep what the caller stored."""
    p = synth.packed_inputs([6, 3, 2], [2, 0, 900], 8, 2, 64, seed=7300, pad_q=5)
    o, lse = run_splitkv(p, CAUSAL, fill=5.0)
    tq = int(p.cu_q[-1])
    assert (o[:4] == 0).all() and np.isneginf(lse[:, :4]).all()          # rows 0..3 of sequence 0
    assert (o[6:9] == 0).all() and np.isneginf(lse[:, 6:9]).all()        # sequence 1 has no keys
    assert (o[tq:] == 5.0).all() and (lse[:, tq:] == 5.0).all()
    check(p, CAUSAL, (o, lse))


@pytest.mark.parametrize("scale", [-0.25, 0.0])
def test_splitkv_scale_sign_and_zero(scale):
    p = synth.packed_inputs([1, 2], [1500, 333], 8, 2, 128, seed=7400)
    check(p, CAUSAL, run_splitkv(p, CAUSAL, scale=scale), scale=scale)
