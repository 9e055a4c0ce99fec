"""Plain CPU fp64 oracle for exact softmax attention (test infrastructure).

THIS IS TEST INFRASTRUCTURE. Only the tests, the smoke check and the CPU
baseline leg of the benchmark may import it. The HIP library never calls it
and shares no code with it.

Pages cited (by title, then section):
  [R] "FlashAttention: exact attention made fast by counting memory traffic"
      (paper review).
  [T] "Flash Attention — Revolutionizing Transformer Efficiency Through
      Memory-Aware Algorithms" (tutorial).
  [C] "FlashAttention and IO-aware exact attention" (curriculum note).

What it computes. The method reaches the plain definition of attention up to
rounding ([R] "The method": the result is exact softmax attention; [T]
"Mathematical Correctness"; [C] "Core ideas"), so the oracle *is* that
definition, in float64, with the score matrix materialised:

    S = scale * Q K^T, with S_ij = -inf where key j is not visible to query i
    LSE_i = m_i + ln sum_j exp(S_ij - m_i),   m_i = max_j S_ij
    P = exp(S - LSE),   O = P V

([T] "The Memory Wall Problem" for S, softmax, PV; [T] "Online Softmax
Algorithm", safe softmax, for the max subtraction; [C] "Core ideas" for
masking before softmax and for the single per-row log-sum-exp.)

The backward pass is not written out on any page ([R] "The method" and
[C] "Core ideas" only say P is recomputed from Q, K, V and the saved row
statistics). The oracle's backward is the derivative of the definition above:

    dV = P^T dO;  dP = dO V^T;  D_i = sum_j P_ij dP_ij;  dS = P * (dP - D)
    dQ = scale * dS K;  dK = scale * dS^T Q

Visibility: mask_kind 0 = every key; 1 = causal (key j visible to query i iff
j <= i + offset, where offset = Nk - Nq aligns the last query with the last
key and is 0 for equal lengths); 2 = block-sparse ([R] "The method",
block-sparse extension): key j visible to query i iff
block_mask[i // block, j // block] != 0, one mask shared by all heads.

Packed variable-length batches and shared K/V heads ([T] "Flash Attention 2
(2023)": variable sequence lengths and multi-/grouped-query attention; [P]
"Implementation: Is It Hard to Adopt?": ragged batches without padding):
sequence b owns query tokens [cu_q[b], cu_q[b+1]) and key tokens
[cu_k[b], cu_k[b+1]) of tensors laid out [tokens, heads, d]; each sequence
is an independent attention problem, and query head h reads K/V head
h // (H // Hkv). The pages give no alignment rule for causal attention with
unequal lengths; the offset above (queries are the last Nq positions of the
key sequence) is the reading taken.

A query row with no visible key has O = 0, LSE = -inf and contributes no
gradient (a user block mask can produce one; so can causal attention with
more queries than keys, and a sequence without keys).

Besides the definition, the module holds the pages' blockwise online
algorithm in float64 (``online_forward_head``, ``online_softmax_row``): it
follows [T] "Block-Wise Attention Computation" and [C] "Core ideas"
(online softmax; tiling and fusion) step by step and is used only to pin the
definition against the algorithm the pages describe.
"""
from __future__ import annotations

import numpy as np

MASK_NONE = 0
MASK_CAUSAL = 1
MASK_BLOCK_SPARSE = 2


# ----------------------------------------------------------------------------
# visibility
# ----------------------------------------------------------------------------
def visible(rows: np.ndarray, N: int, mask_kind: int, block_mask=None, block: int = 128,
            offset: int = 0) -> np.ndarray:
    """Boolean [len(rows), N]: True where key j is visible to query rows[r].

    Causal: [C] "How to approach it" (check with and without a causal mask),
    key j visible to query i iff j <= i + offset; block-sparse: [R] "The
    method" (block-sparse extension).
    """
    rows = np.asarray(rows)
    cols = np.arange(N)
    if mask_kind == MASK_NONE:
        return np.ones((rows.size, N), dtype=bool)
    if mask_kind == MASK_CAUSAL:
        return cols[None, :] <= rows[:, None] + offset
    if mask_kind == MASK_BLOCK_SPARSE:
        bm = np.asarray(block_mask) != 0
        return bm[(rows // block)[:, None], (cols // block)[None, :]]
    raise ValueError(f"unknown mask_kind {mask_kind}")


def _f64(x):
    return np.asarray(x, dtype=np.float64)


# ----------------------------------------------------------------------------
# the definition (one head)
# ----------------------------------------------------------------------------
def causal_offset(nq: int, nk: int) -> int:
    """Causal offset for Nq queries against Nk keys: the last query sees
    every key (Nk - Nq; 0 for equal lengths)."""
    return nk - nq


def _scores(qc, k, scale, rows, N, mask_kind, block_mask, block, offset=0):
    s = scale * (qc @ k.T)
    vis = visible(rows, N, mask_kind, block_mask, block, offset)
    s[~vis] = -np.inf
    return s, vis


def forward_head(q, k, v, scale, mask_kind=MASK_NONE, block_mask=None, rows=None,
                 block: int = 128, chunk: int = 2048, offset=None):
    """O [n, d] and LSE [n] (natural log) of one head for query ``rows``.

    Safe softmax with the row max subtracted ([T] "Online Softmax Algorithm",
    safe softmax) applied to masked, scaled scores; O = P V ([T] "The Memory
    Wall Problem"). ``rows`` defaults to every query; S is materialised for
    ``chunk`` rows at a time. q is [Nq, d], k and v [Nk, d]; the causal
    offset defaults to ``causal_offset(Nq, Nk)``.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    N = k.shape[0]
    offset = causal_offset(q.shape[0], N) if offset is None else offset
    rows = np.arange(q.shape[0]) if rows is None else np.asarray(rows)
    o = np.zeros((rows.size, v.shape[1]))
    lse = np.full(rows.size, -np.inf)
    for c0 in range(0, rows.size, chunk):
        r = rows[c0:c0 + chunk]
        s, vis = _scores(q[r], k, scale, r, N, mask_kind, block_mask, block, offset)
        live = vis.any(axis=1)
        m = np.where(live, s.max(axis=1, initial=-np.inf), 0.0)
        e = np.exp(s - m[:, None])                 # exp(-inf) = 0 on masked keys
        den = e.sum(axis=1)
        with np.errstate(divide="ignore"):
            lse[c0:c0 + r.size] = np.where(live, m + np.log(np.where(live, den, 1.0)), -np.inf)
        p = e / np.where(live, den, 1.0)[:, None]
        o[c0:c0 + r.size] = p @ v
    return o, lse


def probabilities_head(q, k, scale, mask_kind=MASK_NONE, block_mask=None, rows=None, block=128,
                       offset=None):
    """P [n, Nk] of one head (small inputs only; used by the invariant pins)."""
    q, k = _f64(q), _f64(k)
    N = k.shape[0]
    offset = causal_offset(q.shape[0], N) if offset is None else offset
    rows = np.arange(q.shape[0]) if rows is None else np.asarray(rows)
    s, vis = _scores(q[rows], k, scale, rows, N, mask_kind, block_mask, block, offset)
    live = vis.any(axis=1)
    m = np.where(live, s.max(axis=1, initial=-np.inf), 0.0)
    e = np.exp(s - m[:, None])
    den = np.where(live, e.sum(axis=1), 1.0)
    return e / den[:, None]


def backward_head(q, k, v, do, scale, mask_kind=MASK_NONE, block_mask=None,
                  block: int = 128, chunk: int = 2048, offset=None):
    """dQ, dK, dV of one head: the analytic derivative of ``forward_head``.

    P is rebuilt from Q, K and the row log-sum-exp, the same statistics the
    method keeps for its recomputing backward ([R] "The method"; [C] "Core
    ideas", backward by recomputation). The gradient formulas themselves are
    calculus on the definition; no page prints them.
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    Nq, Nk = q.shape[0], k.shape[0]
    offset = causal_offset(Nq, Nk) if offset is None else offset
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for c0 in range(0, Nq, chunk):
        r = np.arange(c0, min(Nq, c0 + chunk))
        s, vis = _scores(q[r], k, scale, r, Nk, mask_kind, block_mask, block, offset)
        live = vis.any(axis=1)
        m = np.where(live, s.max(axis=1, initial=-np.inf), 0.0)
        e = np.exp(s - m[:, None])
        p = e / np.where(live, e.sum(axis=1), 1.0)[:, None]
        doc = do[r]
        dv += p.T @ doc
        dp = doc @ v.T
        dd = (p * dp).sum(axis=1)
        ds = p * (dp - dd[:, None])
        dq[r] = scale * (ds @ k)
        dk += scale * (ds.T @ q[r])
    return dq, dk, dv


def row_term_head(o, do):
    """D_i = sum_k dO_ik O_ik, which equals sum_j P_ij dP_ij (from calculus)."""
    return (_f64(o) * _f64(do)).sum(axis=1)


# ----------------------------------------------------------------------------
# batched wrappers over [B, H, N, d]
# ----------------------------------------------------------------------------
def forward(q, k, v, scale, mask_kind=MASK_NONE, block_mask=None, heads=None, rows=None,
            block: int = 128):
    """Batched ``forward_head``. ``heads`` is a list of (b, h) pairs (default:
    all); returns O [len(heads), n, d] and LSE [len(heads), n]."""
    B, H = q.shape[:2]
    heads = [(b, h) for b in range(B) for h in range(H)] if heads is None else heads
    os_, ls_ = [], []
    for b, h in heads:
        o, l = forward_head(q[b, h], k[b, h], v[b, h], scale, mask_kind, block_mask, rows, block)
        os_.append(o)
        ls_.append(l)
    return np.stack(os_), np.stack(ls_)


def backward(q, k, v, do, scale, mask_kind=MASK_NONE, block_mask=None, heads=None,
             block: int = 128):
    """Batched ``backward_head``; returns dQ, dK, dV stacked over ``heads``."""
    B, H = q.shape[:2]
    heads = [(b, h) for b in range(B) for h in range(H)] if heads is None else heads
    out = [backward_head(q[b, h], k[b, h], v[b, h], do[b, h], scale, mask_kind, block_mask, block)
           for b, h in heads]
    return tuple(np.stack([g[i] for g in out]) for i in range(3))


# ----------------------------------------------------------------------------
# packed variable-length batches with shared K/V heads
# ----------------------------------------------------------------------------
def _spans(cu):
    cu = [int(x) for x in np.asarray(cu)]
    return [(cu[b], cu[b + 1]) for b in range(len(cu) - 1)]


def forward_varlen(q, k, v, cu_q, cu_k, scale, mask_kind=MASK_NONE):
    """Packed batch forward: q [Tq, H, d], k and v [Tk, Hkv, d].

    Sequence b is the ordinary attention problem on its own tokens; query
    head h reads K/V head h // (H // Hkv). Returns O [Tq, H, d] and LSE
    [H, Tq]; tokens outside every sequence keep O = 0 and LSE = -inf.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    Tq, H, d = q.shape
    G = H // k.shape[1]
    o = np.zeros((Tq, H, v.shape[2]))
    lse = np.full((H, Tq), -np.inf)
    for (q0, q1), (k0, k1) in zip(_spans(cu_q), _spans(cu_k)):
        if q1 == q0:
            continue
        for h in range(H):
            ob, lb = forward_head(q[q0:q1, h], k[k0:k1, h // G], v[k0:k1, h // G], scale, mask_kind)
            o[q0:q1, h] = ob
            lse[h, q0:q1] = lb
    return o, lse


def backward_varlen(q, k, v, do, cu_q, cu_k, scale, mask_kind=MASK_NONE):
    """Packed batch backward: dQ [Tq, H, d], dK and dV [Tk, Hkv, d].

    A K/V head's gradients sum the contributions of every query head that
    reads it (the chain rule through the shared operand).
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    H = q.shape[1]
    G = H // k.shape[1]
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for (q0, q1), (k0, k1) in zip(_spans(cu_q), _spans(cu_k)):
        if q1 == q0 or k1 == k0:
            continue
        for h in range(H):
            a, b, c = backward_head(q[q0:q1, h], k[k0:k1, h // G], v[k0:k1, h // G], do[q0:q1, h],
                                    scale, mask_kind)
            dq[q0:q1, h] = a
            dk[k0:k1, h // G] += b
            dv[k0:k1, h // G] += c
    return dq, dk, dv


# ----------------------------------------------------------------------------
# split keys: partial results over key ranges, then the combine rule
# ----------------------------------------------------------------------------
def partial_head(q, k, v, scale, keys, mask_kind=MASK_NONE, offset=None):
    """(O_s, LSE_s) of one head over the key indices ``keys`` only: the
    definition restricted to that range (visibility is still decided by the
    key's position in the whole sequence). A row that sees none of these keys
    gets O_s = 0, LSE_s = -inf."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    keys = np.asarray(keys, dtype=np.int64)
    Nq, Nk = q.shape[0], k.shape[0]
    offset = causal_offset(Nq, Nk) if offset is None else offset
    s = scale * (q @ k[keys].T)
    vis = visible(np.arange(Nq), Nk, mask_kind, offset=offset)[:, keys]
    s[~vis] = -np.inf
    live = vis.any(axis=1)
    m = np.where(live, s.max(axis=1, initial=-np.inf), 0.0)
    e = np.exp(s - m[:, None])
    den = np.where(live, e.sum(axis=1), 1.0)
    o = (e / den[:, None]) @ v[keys]
    with np.errstate(divide="ignore"):
        lse = np.where(live, m + np.log(den), -np.inf)
    return o, lse


def combine_partials(o_parts, lse_parts):
    """Merge per-key-range results of the same rows into the full result.

    The block-combine rule ([T] "Mathematical Correctness": the exponential
    sum of a row is the sum over blocks of each block's sum times
    exp(block max - overall max); [C] "Core ideas": one log-sum-exp per
    row): LSE = max_s LSE_s + ln sum_s exp(LSE_s - max_s LSE_s) and
    O = sum_s exp(LSE_s - LSE) O_s. Ranges a row does not see (LSE_s = -inf)
    weigh 0; a row that sees nothing gets O = 0, LSE = -inf.
    """
    o_parts = [_f64(o) for o in o_parts]
    L = np.stack([_f64(x) for x in lse_parts])           # [S, rows]
    m = L.max(axis=0)
    live = np.isfinite(m)
    ms = np.where(live, m, 0.0)
    w = np.exp(L - ms[None, :])                            # exp(-inf) = 0
    tot = w.sum(axis=0)
    with np.errstate(divide="ignore"):
        lse = np.where(live, ms + np.log(np.where(live, tot, 1.0)), -np.inf)
    wn = w / np.where(live, tot, 1.0)[None, :]
    o = sum(wn[s][:, None] * o_parts[s] for s in range(len(o_parts)))
    return o, lse


# ----------------------------------------------------------------------------
# the pages' blockwise online algorithm (float64), used only to pin the above
# ----------------------------------------------------------------------------
def online_softmax_row(x, values, block_sizes):
    """One query row processed key block by key block.

    Running statistics as in [T] "Online Softmax Algorithm" (online updates)
    and [C] "Core ideas" (online softmax): on each block, m' = max(m, block
    max); the running sum and the unnormalised output are both multiplied by
    exp(m - m') and the block's exp(x - m') terms are added. Dividing the
    output by the sum at the end gives the softmax-weighted value.

    Returns a list of (m, l, o) after each block, then (O, LSE).
    """
    x = _f64(x)
    values = _f64(values)
    m, l = -np.inf, 0.0
    o = np.zeros(values.shape[1:]) if values.ndim > 1 else 0.0
    trace = []
    pos = 0
    for bs in block_sizes:
        xb, vb = x[pos:pos + bs], values[pos:pos + bs]
        pos += bs
        m_new = max(m, float(xb.max()))
        if m_new == -np.inf:                      # nothing visible yet
            trace.append((m, l, o))
            continue
        alpha = np.exp(m - m_new)                 # exp(-inf) = 0 on the first block
        e = np.exp(xb - m_new)
        l = l * alpha + e.sum()
        o = o * alpha + (e @ vb if values.ndim > 1 else float((e * vb).sum()))
        m = m_new
        trace.append((m, l, o))
    assert pos == x.size, "block sizes must cover the row"
    if l == 0.0:
        return trace, (o * 0.0, -np.inf)
    return trace, (o / l, m + np.log(l))


def online_forward_head(q, k, v, scale, mask_kind=MASK_NONE, block_mask=None,
                        q_block: int = 64, k_blocks=None, normalise_each_block: bool = False,
                        block: int = 128):
    """Tiled forward of one head with the online softmax (float64).

    Follows [T] "Block-Wise Attention Computation" (partition Q, K, V into
    blocks; S_ij = Q_i K_j^T on chip; online accumulation) with the rescale
    factor exp(m_old - m_new) on the old accumulator that [C] "Core ideas"
    states, and with [C]'s single per-row log-sum-exp. The query blocks are
    the outer loop and the key blocks the inner one, as in [T] and [C].

    ``k_blocks`` is a list of key-block sizes (default: blocks of q_block).
    ``normalise_each_block`` keeps O normalised after every block (the
    first-version form in [T] "Block-Wise Attention Computation", with the
    exp(m_old - m_new) factor restored) instead of dividing once at the end.
    Returns O [N, d] and LSE [N].
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    N, d = q.shape
    if k_blocks is None:
        k_blocks = [min(q_block, N - s) for s in range(0, N, q_block)]
    assert sum(k_blocks) == N
    o_out = np.zeros((N, v.shape[1]))
    lse_out = np.full(N, -np.inf)
    for i0 in range(0, N, q_block):
        rows = np.arange(i0, min(N, i0 + q_block))
        qi = q[rows]
        m = np.full(rows.size, -np.inf)
        l = np.zeros(rows.size)
        acc = np.zeros((rows.size, v.shape[1]))
        j0 = 0
        for bs in k_blocks:
            cols = np.arange(j0, j0 + bs)
            j0 += bs
            s = scale * (qi @ k[cols].T)
            vis = visible(rows, N, mask_kind, block_mask, block)[:, cols]
            s[~vis] = -np.inf
            m_new = np.maximum(m, s.max(axis=1))
            started = m_new > -np.inf
            m_ref = np.where(started, m_new, 0.0)
            alpha = np.where(started, np.exp(m - m_ref), 0.0)
            p = np.exp(s - m_ref[:, None])
            l_new = alpha * l + p.sum(axis=1)
            if normalise_each_block:
                safe = np.where(l_new > 0, l_new, 1.0)
                acc = ((alpha * l)[:, None] * acc + p @ v[cols]) / safe[:, None]
            else:
                acc = alpha[:, None] * acc + p @ v[cols]
            m, l = m_new, l_new
        live = l > 0
        if normalise_each_block:
            o_out[rows] = np.where(live[:, None], acc, 0.0)
        else:
            o_out[rows] = np.where(live[:, None], acc / np.where(live, l, 1.0)[:, None], 0.0)
        with np.errstate(divide="ignore"):
            lse_out[rows] = np.where(live, m + np.log(np.where(live, l, 1.0)), -np.inf)
    return o_out, lse_out
