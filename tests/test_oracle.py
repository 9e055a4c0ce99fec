"""Pins of the CPU oracle against things other than itself (CPU only).

Each test checks the oracle against something the pages or mathematics fix:
a worked online-softmax example in closed form, the pages' blockwise
algorithm, closed forms, invariances, finite differences and an independent
library routine (torch's float64 scaled_dot_product_attention with autograd).

Pages cited:
  [R] "FlashAttention: exact attention made fast by counting memory traffic".
  [T] "Flash Attention — Revolutionizing Transformer Efficiency Through
      Memory-Aware Algorithms".
  [C] "FlashAttention and IO-aware exact attention".
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import MASK_BLOCK_SPARSE, MASK_CAUSAL, MASK_NONE

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rnd(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


def rand_block_mask(seed, nb, p=0.4, keep_diag=True):
    m = (np.random.default_rng(seed).random((nb, nb)) < p).astype(np.uint8)
    if keep_diag:
        np.fill_diagonal(m, 1)
    return m


# --------------------------------------------------------------------------
# worked online-softmax example: four scores in two blocks of two
# ([T] "Online Softmax Algorithm"; [C] "Core ideas", online softmax).
# The review page mentions such a worked example in a post that is not among
# the pages, so the expected values here are the closed forms of each step.
# --------------------------------------------------------------------------
def test_four_score_online_trace_closed_form():
    x = [1.0, 2.0, 3.0, 4.0]
    v = [1.0, 2.0, 3.0, 4.0]
    trace, (o, lse) = oracle.online_softmax_row(x, v, [2, 2])
    e = math.exp
    # after block {1, 2}: max 2, sum e^-1 + 1, unnormalised output e^-1*1 + 1*2
    m1, l1, o1 = trace[0]
    assert m1 == 2.0
    assert abs(l1 - (e(-1) + 1.0)) < 1e-15
    assert abs(o1 - (e(-1) * 1 + 2.0)) < 1e-15
    # after block {3, 4}: max 4; the old terms are carried by exp(2 - 4)
    m2, l2, o2 = trace[1]
    assert m2 == 4.0
    l2_ref = e(-3) + e(-2) + e(-1) + 1.0
    o2_ref = e(-3) * 1 + e(-2) * 2 + e(-1) * 3 + 4.0
    assert abs(l2 - l2_ref) < 1e-15
    assert abs(o2 - o2_ref) < 1e-14
    assert abs(o - o2_ref / l2_ref) < 1e-15
    assert abs(lse - math.log(e(1) + e(2) + e(3) + e(4))) < 1e-14
    # the same numbers out of the materialising definition
    q = np.array([[1.0]])
    k = np.array([[1.0], [2.0], [3.0], [4.0]])
    vv = np.array([[1.0], [2.0], [3.0], [4.0]])
    # one query against four keys: pad to a square problem with three dummy queries
    qq = np.vstack([q, np.zeros((3, 1))])
    O, L = oracle.forward_head(qq, k, vv, 1.0)
    assert abs(O[0, 0] - o2_ref / l2_ref) < 1e-15
    assert abs(L[0] - math.log(e(1) + e(2) + e(3) + e(4))) < 1e-14
    P = oracle.probabilities_head(qq, k, 1.0)[0]
    den = e(1) + e(2) + e(3) + e(4)
    for j in range(4):
        assert abs(P[j] - e(j + 1) / den) < 1e-15


def test_online_row_any_partition_equals_full_softmax():
    """Block-combine invariant ([T] "Mathematical Correctness"): any split of a
    row into blocks gives the full-row sum of exp(x - max) and the same output."""
    rng = np.random.default_rng(7)
    for trial in range(40):
        n = int(rng.integers(1, 40))
        x = rng.standard_normal(n) * 4
        vals = rng.standard_normal((n, 3))
        cuts = np.sort(rng.choice(np.arange(1, n), size=min(n - 1, int(rng.integers(0, 6))), replace=False)) if n > 1 else []
        sizes = np.diff(np.concatenate([[0], cuts, [n]])).astype(int).tolist()
        _, (o, lse) = oracle.online_softmax_row(x, vals, sizes)
        mx = max(x)
        tot = math.fsum(math.exp(t - mx) for t in x)
        assert abs(lse - (mx + math.log(tot))) < 1e-13
        w = np.array([math.exp(t - mx) / tot for t in x])
        assert np.allclose(o, w @ vals, rtol=0, atol=1e-13)


# --------------------------------------------------------------------------
# blockwise online algorithm == materialising definition, for many tilings
# --------------------------------------------------------------------------
@pytest.mark.parametrize("mask_kind", [MASK_NONE, MASK_CAUSAL, MASK_BLOCK_SPARSE])
def test_blockwise_online_equals_definition(mask_kind):
    N, d = 37, 5
    q, k, v = rnd(1, N, d), rnd(2, N, d), rnd(3, N, d)
    bm = rand_block_mask(4, -(-N // 4)) if mask_kind == MASK_BLOCK_SPARSE else None
    O, L = oracle.forward_head(q, k, v, 0.7, mask_kind, bm, block=4)
    rng = np.random.default_rng(5)
    tilings = [(qb, None) for qb in (1, 2, 5, 16, 37, 64)]
    for _ in range(6):
        cuts = np.sort(rng.choice(np.arange(1, N), size=int(rng.integers(1, 8)), replace=False))
        tilings.append((int(rng.integers(1, N + 1)), np.diff(np.concatenate([[0], cuts, [N]])).tolist()))
    for qb, kbl in tilings:
        for norm in (False, True):
            O2, L2 = oracle.online_forward_head(q, k, v, 0.7, mask_kind, bm, q_block=qb,
                                                k_blocks=kbl, normalise_each_block=norm, block=4)
            assert np.allclose(O2, O, rtol=0, atol=1e-13), (qb, kbl, norm)
            assert np.allclose(L2, L, rtol=0, atol=1e-13), (qb, kbl, norm)


# --------------------------------------------------------------------------
# independent library routine: torch float64 SDPA (+ autograd) on the CPU
# --------------------------------------------------------------------------
def _torch_ref(q, k, v, do, scale, vis):
    tq, tk, tv = (torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(
        tq[None, None], tk[None, None], tv[None, None],
        attn_mask=torch.tensor(vis)[None, None], scale=scale)[0, 0]
    out.backward(torch.tensor(do, dtype=torch.float64))
    s = scale * (tq @ tk.T)
    s = s.masked_fill(~torch.tensor(vis), float("-inf"))
    lse = torch.logsumexp(s, dim=-1)
    return (out.detach().numpy(), lse.detach().numpy(), tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy())


@pytest.mark.parametrize("mask_kind,N,d", [(MASK_NONE, 50, 8), (MASK_CAUSAL, 61, 16),
                                           (MASK_BLOCK_SPARSE, 45, 4), (MASK_NONE, 300, 64),
                                           (MASK_CAUSAL, 200, 128)])
def test_oracle_matches_torch_sdpa_fp64(mask_kind, N, d):
    q, k, v, do = rnd(11, N, d), rnd(12, N, d), rnd(13, N, d), rnd(14, N, d)
    scale = 1.0 / math.sqrt(d)
    blk = 8
    bm = rand_block_mask(15, -(-N // blk)) if mask_kind == MASK_BLOCK_SPARSE else None
    vis = oracle.visible(np.arange(N), N, mask_kind, bm, blk)
    # the visibility itself, written independently of the oracle
    i, j = np.meshgrid(np.arange(N), np.arange(N), indexing="ij")
    if mask_kind == MASK_CAUSAL:
        assert (vis == (j <= i)).all()
    elif mask_kind == MASK_BLOCK_SPARSE:
        assert (vis == (bm[i // blk, j // blk] == 1)).all()
    else:
        assert vis.all()
    ro, rl, rdq, rdk, rdv = _torch_ref(q, k, v, do, scale, vis)
    O, L = oracle.forward_head(q, k, v, scale, mask_kind, bm, block=blk, chunk=17)
    dq, dk, dv = oracle.backward_head(q, k, v, do, scale, mask_kind, bm, block=blk, chunk=23)
    for a, b in ((O, ro), (L, rl), (dq, rdq), (dk, rdk), (dv, rdv)):
        assert np.abs(a - b).max() <= 1e-12 * max(1.0, np.abs(b).max())


# --------------------------------------------------------------------------
# brute-force central finite differences on tiny inputs, every mask kind
# --------------------------------------------------------------------------
@pytest.mark.parametrize("mask_kind", [MASK_NONE, MASK_CAUSAL, MASK_BLOCK_SPARSE])
def test_backward_matches_finite_differences(mask_kind):
    N, d = 7, 3
    q, k, v, g = rnd(21, N, d), rnd(22, N, d), rnd(23, N, d), rnd(24, N, d)
    bm = rand_block_mask(25, 4, p=0.5) if mask_kind == MASK_BLOCK_SPARSE else None
    scale = 0.8

    def loss(qq, kk, vv):
        O, _ = oracle.forward_head(qq, kk, vv, scale, mask_kind, bm, block=2)
        return float((O * g).sum())

    dq, dk, dv = oracle.backward_head(q, k, v, g, scale, mask_kind, bm, block=2)
    h = 1e-5
    for which, grad in ((0, dq), (1, dk), (2, dv)):
        num = np.zeros_like(grad)
        for idx in np.ndindex(*grad.shape):
            args_p = [q.copy(), k.copy(), v.copy()]
            args_m = [q.copy(), k.copy(), v.copy()]
            args_p[which][idx] += h
            args_m[which][idx] -= h
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        assert np.abs(num - grad).max() <= 1e-8 * max(1.0, np.abs(grad).max()), which


# --------------------------------------------------------------------------
# closed forms
# --------------------------------------------------------------------------
@pytest.mark.parametrize("mask_kind", [MASK_NONE, MASK_CAUSAL, MASK_BLOCK_SPARSE])
def test_zero_queries_give_uniform_attention(mask_kind):
    """Q = 0: every visible score is 0, so O_i is the mean of the visible V
    rows and LSE_i = ln(number of visible keys)."""
    N, d = 40, 6
    v = rnd(31, N, d)
    bm = rand_block_mask(32, 10) if mask_kind == MASK_BLOCK_SPARSE else None
    O, L = oracle.forward_head(np.zeros((N, d)), rnd(33, N, d), v, 0.5, mask_kind, bm, block=4)
    for i in range(N):
        if mask_kind == MASK_NONE:
            cols = np.arange(N)
        elif mask_kind == MASK_CAUSAL:
            cols = np.arange(i + 1)                # prefix: keys 0..i
        else:
            cols = np.array([j for j in range(N) if bm[i // 4, j // 4]])
        assert abs(L[i] - math.log(cols.size)) < 1e-13
        assert np.allclose(O[i], v[cols].mean(axis=0), rtol=0, atol=1e-13)


def test_constant_values_and_single_key():
    N, d = 33, 5
    q, k = rnd(41, N, d), rnd(42, N, d)
    vrow = rnd(43, d)
    for mk in (MASK_NONE, MASK_CAUSAL):
        O, _ = oracle.forward_head(q, k, np.tile(vrow, (N, 1)), 0.3, mk)
        assert np.allclose(O, vrow[None, :], rtol=0, atol=1e-13)
    # causal row 0 sees only key 0
    v = rnd(44, N, d)
    O, L = oracle.forward_head(q, k, v, 0.3, MASK_CAUSAL)
    assert np.allclose(O[0], v[0], rtol=0, atol=1e-15)
    assert abs(L[0] - 0.3 * float(q[0] @ k[0])) < 1e-14


def test_rows_of_p_sum_to_one_and_p_matches_exp_s_minus_lse():
    N, d = 29, 4
    q, k = rnd(51, N, d), rnd(52, N, d)
    for mk in (MASK_NONE, MASK_CAUSAL):
        P = oracle.probabilities_head(q, k, 0.9, mk)
        assert np.allclose(P.sum(axis=1), 1.0, rtol=0, atol=1e-14)
        _, L = oracle.forward_head(q, k, rnd(53, N, d), 0.9, mk)
        s = 0.9 * q @ k.T
        vis = oracle.visible(np.arange(N), N, mk)
        assert np.allclose(np.where(vis, np.exp(s - L[:, None]), 0.0), P, rtol=0, atol=1e-14)


# --------------------------------------------------------------------------
# invariances
# --------------------------------------------------------------------------
def test_invariances():
    N, d = 31, 6
    q, k, v = rnd(61, N, d), rnd(62, N, d), rnd(63, N, d)
    O, L = oracle.forward_head(q, k, v, 0.4)
    # (Q * c, scale / c)
    O2, L2 = oracle.forward_head(q * 2.5, k, v, 0.4 / 2.5)
    assert np.allclose(O2, O, atol=1e-13) and np.allclose(L2, L, atol=1e-13)
    # shifting every key by one vector shifts each row's scores by a constant
    shift = rnd(64, d)
    O3, L3 = oracle.forward_head(q, k + shift, v, 0.4)
    assert np.allclose(O3, O, atol=1e-12)
    assert np.allclose(L3, L + 0.4 * q @ shift, atol=1e-12)
    # joint permutation of keys/values leaves O unchanged; permuting queries permutes O
    perm = np.random.default_rng(65).permutation(N)
    O4, L4 = oracle.forward_head(q, k[perm], v[perm], 0.4)
    assert np.allclose(O4, O, atol=1e-13) and np.allclose(L4, L, atol=1e-13)
    O5, L5 = oracle.forward_head(q[perm], k, v, 0.4)
    assert np.allclose(O5, O[perm], atol=1e-13) and np.allclose(L5, L[perm], atol=1e-13)


# --------------------------------------------------------------------------
# mask special cases
# --------------------------------------------------------------------------
def test_block_mask_special_cases():
    N, d, blk = 24, 4, 6
    q, k, v, do = rnd(71, N, d), rnd(72, N, d), rnd(73, N, d), rnd(74, N, d)
    nb = N // blk
    ones = np.ones((nb, nb), np.uint8)
    O, L = oracle.forward_head(q, k, v, 0.5, MASK_BLOCK_SPARSE, ones, block=blk)
    Or, Lr = oracle.forward_head(q, k, v, 0.5, MASK_NONE)
    assert np.allclose(O, Or, atol=1e-14) and np.allclose(L, Lr, atol=1e-14)
    g1 = oracle.backward_head(q, k, v, do, 0.5, MASK_BLOCK_SPARSE, ones, block=blk)
    g2 = oracle.backward_head(q, k, v, do, 0.5, MASK_NONE)
    for a, b in zip(g1, g2):
        assert np.allclose(a, b, atol=1e-13)
    # diagonal-only mask == independent dense attention per block
    diag = np.eye(nb, dtype=np.uint8)
    O, L = oracle.forward_head(q, k, v, 0.5, MASK_BLOCK_SPARSE, diag, block=blk)
    for b in range(nb):
        sl = slice(b * blk, (b + 1) * blk)
        Ob, Lb = oracle.forward_head(q[sl], k[sl], v[sl], 0.5)
        assert np.allclose(O[sl], Ob, atol=1e-14) and np.allclose(L[sl], Lb, atol=1e-14)


def test_empty_rows():
    """A query block whose mask row is empty: O = 0, LSE = -inf, no gradient."""
    N, d, blk = 12, 3, 4
    q, k, v, do = rnd(81, N, d), rnd(82, N, d), rnd(83, N, d), rnd(84, N, d)
    bm = np.array([[1, 0, 1], [0, 0, 0], [1, 1, 1]], np.uint8)
    O, L = oracle.forward_head(q, k, v, 0.5, MASK_BLOCK_SPARSE, bm, block=blk)
    assert (O[4:8] == 0).all() and np.isneginf(L[4:8]).all()
    assert np.isfinite(L[:4]).all() and np.isfinite(L[8:]).all()
    dq, dk, dv = oracle.backward_head(q, k, v, do, 0.5, MASK_BLOCK_SPARSE, bm, block=blk)
    assert (dq[4:8] == 0).all()
    # the empty rows must not leak into dK/dV: zeroing their dO changes nothing
    do2 = do.copy()
    do2[4:8] = 123.0
    _, dk2, dv2 = oracle.backward_head(q, k, v, do2, 0.5, MASK_BLOCK_SPARSE, bm, block=blk)
    assert np.array_equal(dk, dk2) and np.array_equal(dv, dv2)
    O2, _ = oracle.online_forward_head(q, k, v, 0.5, MASK_BLOCK_SPARSE, bm, q_block=4, block=blk)
    assert np.allclose(O2, O, atol=1e-14)


# --------------------------------------------------------------------------
# backward identities
# --------------------------------------------------------------------------
@pytest.mark.parametrize("mask_kind", [MASK_NONE, MASK_CAUSAL, MASK_BLOCK_SPARSE])
def test_backward_identities(mask_kind):
    N, d = 36, 5
    q, k, v, do = rnd(91, N, d), rnd(92, N, d), rnd(93, N, d), rnd(94, N, d)
    bm = rand_block_mask(95, 9) if mask_kind == MASK_BLOCK_SPARSE else None
    sc = 0.6
    dq, dk, dv = oracle.backward_head(q, k, v, do, sc, mask_kind, bm, block=4)
    # rows of P sum to one: column sums of dV equal column sums of dO
    assert np.allclose(dv.sum(axis=0), do.sum(axis=0), atol=1e-12)
    # shift invariance in K: the dK rows sum to zero
    assert np.allclose(dk.sum(axis=0), 0.0, atol=1e-12)
    # S is bilinear in (Q, K): <dQ, Q> = <dK, K>
    assert abs((dq * q).sum() - (dk * k).sum()) < 1e-11
    # D_i = rowsum(dO * O) = rowsum(P * dP)
    O, _ = oracle.forward_head(q, k, v, sc, mask_kind, bm, block=4)
    P = oracle.probabilities_head(q, k, sc, mask_kind, bm, block=4)
    assert np.allclose(oracle.row_term_head(O, do), (P * (do @ v.T)).sum(axis=1), atol=1e-12)
    # constant V: O does not depend on Q or K
    vc = np.tile(rnd(96, d), (N, 1))
    dq0, dk0, _ = oracle.backward_head(q, k, vc, do, sc, mask_kind, bm, block=4)
    assert np.abs(dq0).max() < 1e-13 and np.abs(dk0).max() < 1e-13


# --------------------------------------------------------------------------
# the pages' attention-matrix memory table (golden fixture)
# --------------------------------------------------------------------------
def test_attention_matrix_memory_table():
    tab = json.load(open(os.path.join(GOLDEN, "attention_matrix_memory.json")))
    unit = {"K": 2 ** 10, "M": 2 ** 20, "B": 2 ** 30, "MB": 2 ** 20, "GB": 2 ** 30}

    def parse(s):
        s = s.replace(" ", "")
        for suf in ("MB", "GB", "K", "M", "B"):
            if s.endswith(suf):
                return int(s[: -len(suf)]) * unit[suf]
        return int(s)

    for row in tab["rows"]:
        N = row["N"]
        assert parse(row["seq"]) == N
        assert parse(row["elements"]) == N * N
        assert parse(row["fp32"]) == 4 * N * N
        assert parse(row["fp16"]) == 2 * N * N
    # the oracle materialises exactly N x N probabilities per head (2K row)
    P = oracle.probabilities_head(np.zeros((2048, 1)), np.zeros((2048, 1)), 1.0)
    assert P.size == parse(tab["rows"][0]["elements"])
    assert P.astype(np.float32).nbytes == parse(tab["rows"][0]["fp32"])


# --------------------------------------------------------------------------
# unequal lengths, shared K/V heads and packed batches ([T] "Flash Attention 2
# (2023)"; [P] "Implementation: Is It Hard to Adopt?"), pinned against torch's
# float64 SDPA + autograd with masks built here, independently of the oracle
# --------------------------------------------------------------------------
def _sdpa_grads(q, k, v, do, scale, vis):
    """q [H, Nq, d], k, v [Hkv, Nk, d] (repeated per group inside torch, so
    autograd sums the group's contributions); vis [Nq, Nk] bool."""
    H, Hkv = q.shape[0], k.shape[0]
    tq, tk, tv = (torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (q, k, v))
    kk = tk.repeat_interleave(H // Hkv, dim=0)
    vv = tv.repeat_interleave(H // Hkv, dim=0)
    m = torch.tensor(vis)
    out = torch.nn.functional.scaled_dot_product_attention(tq[None], kk[None], vv[None],
                                                           attn_mask=m[None, None], scale=scale)[0]
    out.backward(torch.tensor(do, dtype=torch.float64))
    s = (scale * (tq @ kk.transpose(1, 2))).masked_fill(~m, float("-inf"))
    lse = torch.logsumexp(s, dim=-1)
    return [x.detach().numpy() for x in (out, lse, tq.grad, tk.grad, tv.grad)]


@pytest.mark.parametrize("nq,nk", [(5, 23), (17, 17), (1, 40), (31, 64)])
def test_causal_offset_matches_bottom_right_sdpa(nq, nk):
    """Nq <= Nk: query i sees keys 0 .. i + Nk - Nq (the last query sees all)."""
    d, sc = 6, 0.45
    q, k, v, do = rnd(201, 1, nq, d), rnd(202, 1, nk, d), rnd(203, 1, nk, d), rnd(204, 1, nq, d)
    vis = np.tril(np.ones((nq, nk), bool), k=nk - nq)
    assert vis[-1].all() and vis[0].sum() == nk - nq + 1
    ro, rl, rdq, rdk, rdv = _sdpa_grads(q, k, v, do, sc, vis)
    O, L = oracle.forward_head(q[0], k[0], v[0], sc, MASK_CAUSAL, chunk=4)
    dq, dk, dv = oracle.backward_head(q[0], k[0], v[0], do[0], sc, MASK_CAUSAL, chunk=3)
    for a, b in ((O, ro[0]), (L, rl[0]), (dq, rdq[0]), (dk, rdk[0]), (dv, rdv[0])):
        assert np.abs(a - b).max() <= 1e-12 * max(1.0, np.abs(b).max())
    # the same numbers as the last Nq rows of the square causal problem
    qf = np.vstack([rnd(205, nk - nq, d), q[0]])
    Of, Lf = oracle.forward_head(qf, k[0], v[0], sc, MASK_CAUSAL)
    assert np.allclose(O, Of[nk - nq:], rtol=0, atol=1e-13)
    assert np.allclose(L, Lf[nk - nq:], rtol=0, atol=1e-13)


def test_causal_offset_more_queries_than_keys():
    """Nq > Nk: the first Nq - Nk queries see no key (O = 0, LSE = -inf, no
    gradient); the rest match the bottom-right SDPA."""
    nq, nk, d, sc = 20, 12, 5, 0.7
    q, k, v, do = rnd(211, nq, d), rnd(212, nk, d), rnd(213, nk, d), rnd(214, nq, d)
    O, L = oracle.forward_head(q, k, v, sc, MASK_CAUSAL)
    dq, dk, dv = oracle.backward_head(q, k, v, do, sc, MASK_CAUSAL)
    e = nq - nk
    assert (O[:e] == 0).all() and np.isneginf(L[:e]).all() and (dq[:e] == 0).all()
    vis = np.tril(np.ones((nk, nk), bool))
    ro, rl, rdq, rdk, rdv = _sdpa_grads(q[None, e:], k[None], v[None], do[None, e:], sc, vis)
    for a, b in ((O[e:], ro[0]), (L[e:], rl[0]), (dq[e:], rdq[0]), (dk, rdk[0]), (dv, rdv[0])):
        assert np.abs(a - b).max() <= 1e-12 * max(1.0, np.abs(b).max())


@pytest.mark.parametrize("H,Hkv", [(4, 2), (6, 1), (3, 3)])
@pytest.mark.parametrize("mask_kind", [MASK_NONE, MASK_CAUSAL])
def test_varlen_gqa_matches_per_sequence_sdpa(H, Hkv, mask_kind):
    """Packed [tokens, heads, d] batches with K/V heads shared by groups of
    query heads: each sequence against torch SDPA on that sequence alone."""
    d, sc = 8, 0.35
    lq, lk = [7, 1, 19, 0, 12], [7, 9, 25, 4, 12]
    if mask_kind == MASK_NONE:
        lk = [7, 9, 3, 4, 12]
    cu_q, cu_k = np.concatenate([[0], np.cumsum(lq)]), np.concatenate([[0], np.cumsum(lk)])
    Tq, Tk = int(cu_q[-1]), int(cu_k[-1])
    q, k, v, do = rnd(221, Tq, H, d), rnd(222, Tk, Hkv, d), rnd(223, Tk, Hkv, d), rnd(224, Tq, H, d)
    O, L = oracle.forward_varlen(q, k, v, cu_q, cu_k, sc, mask_kind)
    dq, dk, dv = oracle.backward_varlen(q, k, v, do, cu_q, cu_k, sc, mask_kind)
    assert O.shape == (Tq, H, d) and L.shape == (H, Tq) and dk.shape == (Tk, Hkv, d)
    for b in range(len(lq)):
        qs, ks = slice(cu_q[b], cu_q[b + 1]), slice(cu_k[b], cu_k[b + 1])
        if lq[b] == 0:
            assert (dk[ks] == 0).all() and (dv[ks] == 0).all()
            continue
        vis = np.ones((lq[b], lk[b]), bool)
        if mask_kind == MASK_CAUSAL:
            vis = np.tril(vis, k=lk[b] - lq[b])
        t = lambda a, s: np.ascontiguousarray(a[s].transpose(1, 0, 2))
        ro, rl, rdq, rdk, rdv = _sdpa_grads(t(q, qs), t(k, ks), t(v, ks), t(do, qs), sc, vis)
        for a, r in ((t(O, qs), ro), (L[:, qs], rl), (t(dq, qs), rdq), (t(dk, ks), rdk), (t(dv, ks), rdv)):
            assert np.abs(a - r).max() <= 1e-12 * max(1.0, np.abs(r).max()), b


def test_varlen_single_sequence_equals_dense_heads():
    """One packed sequence with Hkv = H is the dense per-head problem."""
    N, H, d, sc = 21, 3, 4, 0.6
    q, k, v = rnd(231, N, H, d), rnd(232, N, H, d), rnd(233, N, H, d)
    O, L = oracle.forward_varlen(q, k, v, [0, N], [0, N], sc, MASK_CAUSAL)
    for h in range(H):
        Oh, Lh = oracle.forward_head(q[:, h], k[:, h], v[:, h], sc, MASK_CAUSAL)
        assert np.array_equal(O[:, h], Oh) and np.array_equal(L[h], Lh)


# --------------------------------------------------------------------------
# key ranges computed apart and merged with the block-combine rule
# ([T] "Mathematical Correctness"; [C] "Core ideas")
# --------------------------------------------------------------------------
def test_combine_two_single_key_ranges_closed_form():
    """One query, keys with scores a and b in two ranges: the merged LSE is
    ln(e^a + e^b) and O the softmax-weighted mix of the two values."""
    a, b = 0.3, -1.7
    o, lse = oracle.combine_partials([np.array([[2.0]]), np.array([[-5.0]])], [np.array([a]), np.array([b])])
    assert abs(lse[0] - math.log(math.exp(a) + math.exp(b))) < 1e-15
    wa = math.exp(a) / (math.exp(a) + math.exp(b))
    assert abs(o[0, 0] - (wa * 2.0 + (1 - wa) * -5.0)) < 1e-15


@pytest.mark.parametrize("mask_kind", [MASK_NONE, MASK_CAUSAL])
def test_split_key_ranges_combine_to_the_definition(mask_kind):
    rng = np.random.default_rng(301)
    for nq, nk in ((1, 200), (5, 97), (16, 300), (20, 12)):
        d = 7
        q, k, v = rnd(302, nq, d), rnd(303, nk, d), rnd(304, nk, d)
        O, L = oracle.forward_head(q, k, v, 0.6, mask_kind)
        for _ in range(4):
            cuts = np.sort(rng.choice(np.arange(1, nk), size=int(rng.integers(0, min(9, nk - 1))), replace=False))
            bounds = np.concatenate([[0], cuts, [nk]]).astype(int)
            parts = [oracle.partial_head(q, k, v, 0.6, np.arange(bounds[i], bounds[i + 1]), mask_kind)
                     for i in range(len(bounds) - 1)]
            o, lse = oracle.combine_partials([x[0] for x in parts], [x[1] for x in parts])
            assert np.allclose(o, O, rtol=0, atol=1e-13)
            fin = np.isfinite(L)
            assert (np.isfinite(lse) == fin).all() and np.allclose(lse[fin], L[fin], rtol=0, atol=1e-13)


def test_combine_with_empty_ranges():
    """A range no row sees weighs nothing; all ranges empty -> O = 0, LSE = -inf."""
    nq, nk, d = 3, 40, 4
    q, k, v = rnd(311, nq, d), rnd(312, nk, d), rnd(313, nk, d)
    O, L = oracle.forward_head(q, k, v, 0.9, MASK_NONE)
    full = oracle.partial_head(q, k, v, 0.9, np.arange(nk))
    empty = oracle.partial_head(q, k, v, 0.9, np.arange(0))
    assert (empty[0] == 0).all() and np.isneginf(empty[1]).all()
    o, lse = oracle.combine_partials([empty[0], full[0], empty[0]], [empty[1], full[1], empty[1]])
    assert np.allclose(o, O, atol=1e-14) and np.allclose(lse, L, atol=1e-14)
    o, lse = oracle.combine_partials([empty[0]] * 2, [empty[1]] * 2)
    assert (o == 0).all() and np.isneginf(lse).all()


def test_no_keys_at_all():
    """Zero keys: every row is empty (O = 0, LSE = -inf, no gradient), the
    same convention as a fully masked row."""
    q, do = rnd(321, 3, 4), rnd(322, 3, 4)
    k = v = np.zeros((0, 4))
    for mk in (MASK_NONE, MASK_CAUSAL):
        O, L = oracle.forward_head(q, k, v, 0.5, mk)
        assert O.shape == (3, 4) and (O == 0).all() and np.isneginf(L).all()
        dq, dk, dv = oracle.backward_head(q, k, v, do, 0.5, mk)
        assert (dq == 0).all() and dk.shape == (0, 4) and dv.shape == (0, 4)
    O, L = oracle.forward_varlen(rnd(323, 2, 2, 4), np.zeros((0, 1, 4)), np.zeros((0, 1, 4)), [0, 2], [0, 0], 0.5)
    assert (O == 0).all() and np.isneginf(L).all()


# --------------------------------------------------------------------------
# batched wrappers and the sampled-rows path, against torch float64 SDPA run
# over whole [B, H, N, d] tensors (torch handles the batch and head axes
# itself, so a (b, h) ordering slip in the oracle's stacking shows up)
# --------------------------------------------------------------------------
def _vis_independent(nq, nk, mask_kind, bm, blk, offset=0):
    """Visibility written out from the mask definitions, not via the oracle."""
    i, j = np.meshgrid(np.arange(nq), np.arange(nk), indexing="ij")
    if mask_kind == MASK_CAUSAL:
        return j <= i + offset
    if mask_kind == MASK_BLOCK_SPARSE:
        return bm[i // blk, j // blk] != 0
    return np.ones((nq, nk), dtype=bool)


def _torch_ref_batched(q, k, v, do, scale, vis):
    tq, tk, tv = (torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (q, k, v))
    m = torch.tensor(vis)
    out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=m, scale=scale)
    out.backward(torch.tensor(do, dtype=torch.float64))
    s = (scale * (tq @ tk.transpose(-1, -2))).masked_fill(~m, float("-inf"))
    lse = torch.logsumexp(s, dim=-1)
    return (out.detach().numpy(), lse.detach().numpy(), tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy())


@pytest.mark.parametrize("mask_kind", [MASK_NONE, MASK_CAUSAL, MASK_BLOCK_SPARSE])
def test_batched_wrappers_match_sdpa_over_batch_and_heads(mask_kind):
    """oracle.forward / oracle.backward stack their heads in (b, h) order,
    h fastest, and a ``heads`` list selects and orders them. B != H (both
    > 1) and every head holds different numbers, so a swapped or shifted
    head index fails."""
    B, H, N, d, blk = 2, 3, 19, 4, 4
    rng = np.random.default_rng(41)
    q, k, v, do = (rng.standard_normal((B, H, N, d)) for _ in range(4))
    bm = rand_block_mask(42, -(-N // blk)) if mask_kind == MASK_BLOCK_SPARSE else None
    scale = 0.6
    vis = _vis_independent(N, N, mask_kind, bm, blk)
    ro, rl, rdq, rdk, rdv = _torch_ref_batched(q, k, v, do, scale, vis)
    O, L = oracle.forward(q, k, v, scale, mask_kind, bm, block=blk)
    dq, dk, dv = oracle.backward(q, k, v, do, scale, mask_kind, bm, block=blk)
    assert O.shape == (B * H, N, d) and L.shape == (B * H, N)
    for a, b in ((O, ro), (L, rl), (dq, rdq), (dk, rdk), (dv, rdv)):
        assert np.abs(a - b.reshape(a.shape)).max() <= 1e-12 * max(1.0, np.abs(b).max())
    heads = [(1, 2), (0, 0), (1, 0), (0, 2)]
    O2, L2 = oracle.forward(q, k, v, scale, mask_kind, bm, heads=heads, block=blk)
    g2 = oracle.backward(q, k, v, do, scale, mask_kind, bm, heads=heads, block=blk)
    for i, (b, h) in enumerate(heads):
        assert np.abs(O2[i] - ro[b, h]).max() <= 1e-12
        assert np.abs(L2[i] - rl[b, h]).max() <= 1e-12
        for g, ref in zip(g2, (rdq, rdk, rdv)):
            assert np.abs(g[i] - ref[b, h]).max() <= 1e-12 * max(1.0, np.abs(ref).max())
    # a row sample through the batched wrapper: same rows of every selected head
    rows = np.array([17, 3, 11, 0, 18])
    O3, L3 = oracle.forward(q, k, v, scale, mask_kind, bm, heads=heads, rows=rows, block=blk)
    for i, (b, h) in enumerate(heads):
        assert np.abs(O3[i] - ro[b, h][rows]).max() <= 1e-12
        assert np.abs(L3[i] - rl[b, h][rows]).max() <= 1e-12


@pytest.mark.parametrize("case", ["none", "causal", "block_sparse", "causal_offset"])
def test_forward_head_row_sample_equals_full_rows(case):
    """forward_head(rows=...) on a shuffled, duplicate-free row sample that
    crosses several ``chunk`` boundaries gives exactly the sampled rows of
    the full result, in sample order. Visibility must follow each row's
    position in the sequence (not in the sample) and each chunk's LSE must
    land in its own slots; SDPA on the full problem pins both."""
    mask_kind = {"none": MASK_NONE, "causal": MASK_CAUSAL, "block_sparse": MASK_BLOCK_SPARSE,
                 "causal_offset": MASK_CAUSAL}[case]
    nq, nk, d, blk = (37, 53, 6, 8) if case == "causal_offset" else (45, 45, 6, 8)
    rng = np.random.default_rng(43)
    q, do = rng.standard_normal((nq, d)), rng.standard_normal((nq, d))
    k, v = rng.standard_normal((nk, d)), rng.standard_normal((nk, d))
    bm = rand_block_mask(44, -(-nk // blk)) if mask_kind == MASK_BLOCK_SPARSE else None
    scale = 0.9
    offset = nk - nq
    vis = _vis_independent(nq, nk, mask_kind, bm, blk, offset)
    ro, rl, _, _, _ = _torch_ref_batched(q, k, v, do, scale, vis)
    rows = rng.permutation(nq)[:29]
    assert len(set(rows.tolist())) == rows.size and not (np.diff(rows) > 0).all()
    Of, Lf = oracle.forward_head(q, k, v, scale, mask_kind, bm, block=blk)
    for chunk in (1, 6, 7, 29, 2048):
        Os, Ls = oracle.forward_head(q, k, v, scale, mask_kind, bm, rows=rows, block=blk, chunk=chunk)
        assert Os.shape == (rows.size, d) and Ls.shape == (rows.size,)
        assert np.abs(Os - ro[rows]).max() <= 1e-12, chunk
        assert np.abs(Ls - rl[rows]).max() <= 1e-12, chunk
        assert np.abs(Os - Of[rows]).max() <= 1e-13 and np.abs(Ls - Lf[rows]).max() <= 1e-13
