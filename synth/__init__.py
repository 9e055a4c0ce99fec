"""Seeded synthetic inputs shared by the CPU oracle and the HIP path.

This module only *draws* inputs. It holds none of the attention arithmetic:
no scores, no softmax, no products. Both sides of every parity check take
their inputs from here, so they see bit-identical values.

Recipe (the pages give no generator, so this is a stated choice):

* ``numpy.random.default_rng(seed)``; ``standard_normal(dtype=float32)``
  drawn in the order Q, K, V, dO, each of shape [B, H, N, d]
  (the [N, d]-per-head layout of the tutorial page "Flash Attention —
  Revolutionizing Transformer Efficiency Through Memory-Aware Algorithms",
  section "The Memory Wall Problem").
* bf16 inputs are the fp32 draws rounded to nearest, ties to even, on the
  fp32 bit pattern. The fp32 value of those bf16 bits is what the oracle
  receives, so both sides see the same numbers.
* The block-sparse mask (the review page "FlashAttention: exact attention
  made fast by counting memory traffic", section "The method", extension to
  block-sparse attention) is one uint8 matrix of 128 x 128 blocks shared by
  every (batch, head): diagonal blocks always kept, every off-diagonal block
  kept independently with probability 0.25, drawn from
  ``default_rng(100 + seed).random((nb, nb)) < 0.25``.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

MASK_NONE = 0
MASK_CAUSAL = 1
MASK_BLOCK_SPARSE = 2
MASK_BLOCK = 128          # granularity of the block-sparse mask, in rows/cols

DTYPE_BF16 = 0
DTYPE_F32 = 1


@dataclasses.dataclass(frozen=True)
class Workload:
    """One attention workload: shape, dtype, mask kind and seed."""
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: int          # DTYPE_BF16 or DTYPE_F32
    mask_kind: int      # MASK_NONE / MASK_CAUSAL / MASK_BLOCK_SPARSE
    backward: bool      # whether the workload includes the backward pass
    seed: int

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)


# The five workloads the build is measured and checked on.
WORKLOADS = {
    "tiny_f32": Workload("tiny_f32", 1, 1, 128, 64, DTYPE_F32, MASK_NONE, True, 1),
    "gpt2_medium": Workload("gpt2_medium", 64, 16, 1024, 64, DTYPE_BF16, MASK_NONE, True, 2),
    "causal_train": Workload("causal_train", 8, 16, 4096, 128, DTYPE_BF16, MASK_CAUSAL, True, 3),
    "long_prefill": Workload("long_prefill", 1, 32, 32768, 128, DTYPE_BF16, MASK_CAUSAL, False, 4),
    "block_sparse": Workload("block_sparse", 16, 16, 4096, 64, DTYPE_BF16, MASK_BLOCK_SPARSE, True, 5),
}


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest, ties to even.

    NaN stays NaN (quiet), +-inf and values that round past the largest
    finite bf16 become +-inf, subnormals round like any other value.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint32)
    nan = np.isnan(x)
    if nan.any():
        r = np.where(nan, ((u >> 16) | 0x40).astype(np.uint32), r)
    return r.astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> their exact fp32 values."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def normal_tensors(seed: int, shape, count: int) -> list[np.ndarray]:
    """``count`` fp32 N(0,1) arrays of ``shape`` drawn in order from ``seed``."""
    rng = np.random.default_rng(seed)
    return [rng.standard_normal(shape, dtype=np.float32) for _ in range(count)]


def block_mask(N: int, seed: int, p: float = 0.25, block: int = MASK_BLOCK) -> np.ndarray:
    """uint8 [nb, nb] keep-mask, nb = ceil(N / block); diagonal forced to 1."""
    nb = -(-N // block)
    rng = np.random.default_rng(100 + seed)
    m = (rng.random((nb, nb)) < p).astype(np.uint8)
    np.fill_diagonal(m, 1)
    return m


@dataclasses.dataclass
class Inputs:
    """Inputs of one workload.

    ``q, k, v, do`` are fp32 arrays holding exactly the values the GPU sees
    (for bf16 they are the bf16-rounded draws). ``*_bits`` are the uint16
    bf16 patterns (None for fp32 workloads). ``mask`` is the uint8 block mask
    or None.
    """
    w: Workload
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    do: np.ndarray | None
    q_bits: np.ndarray | None = None
    k_bits: np.ndarray | None = None
    v_bits: np.ndarray | None = None
    do_bits: np.ndarray | None = None
    mask: np.ndarray | None = None


def make_inputs(w: Workload, seed: int | None = None, with_do: bool | None = None) -> Inputs:
    """Draw the inputs of workload ``w`` (seed defaults to ``w.seed``)."""
    seed = w.seed if seed is None else seed
    with_do = w.backward if with_do is None else with_do
    shape = (w.B, w.H, w.N, w.d)
    arrs = normal_tensors(seed, shape, 4 if with_do else 3)
    mask = block_mask(w.N, seed) if w.mask_kind == MASK_BLOCK_SPARSE else None
    if w.dtype == DTYPE_F32:
        q, k, v = arrs[:3]
        do = arrs[3] if with_do else None
        return Inputs(w, q, k, v, do, mask=mask)
    bits = [bf16_bits(a) for a in arrs]
    del arrs
    vals = [bf16_to_f32(b) for b in bits]
    return Inputs(w, vals[0], vals[1], vals[2], vals[3] if with_do else None,
                  bits[0], bits[1], bits[2], bits[3] if with_do else None, mask=mask)


def small_workload(B, H, N, d, dtype=DTYPE_BF16, mask_kind=MASK_NONE, seed=0, backward=True):
    """A workload of arbitrary shape for parity cases (ragged N, tiny B, H)."""
    return Workload(f"B{B}H{H}N{N}d{d}", B, H, N, d, dtype, mask_kind, backward, seed)


# ---------------------------------------------------------------------------
# packed variable-length batches (tokens of all sequences back to back)
# ---------------------------------------------------------------------------
@dataclasses.dataclass
class PackedInputs:
    """A packed batch: q, do [total_q, H, d]; k, v [total_k, Hkv, d].

    ``cu_q`` / ``cu_k`` are the int32 cumulative offsets (B + 1 entries);
    tokens past ``cu_q[-1]`` / ``cu_k[-1]`` (``pad_q`` / ``pad_k`` of them)
    belong to no sequence. Values are bf16-rounded fp32 as in ``Inputs``.
    """
    lens_q: list
    lens_k: list
    H: int
    Hkv: int
    d: int
    seed: int
    cu_q: np.ndarray
    cu_k: np.ndarray
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    do: np.ndarray
    q_bits: np.ndarray
    k_bits: np.ndarray
    v_bits: np.ndarray
    do_bits: np.ndarray

    @property
    def B(self) -> int:
        return len(self.lens_q)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def name(self) -> str:
        return f"packed B{self.B} H{self.H}/{self.Hkv} d{self.d} Tq{self.q.shape[0]} Tk{self.k.shape[0]}"


def offsets(lens) -> np.ndarray:
    """int32 [len(lens) + 1] cumulative token offsets starting at 0."""
    return np.concatenate([[0], np.cumsum(np.asarray(lens, dtype=np.int64))]).astype(np.int32)


def packed_inputs(lens_q, lens_k, H, Hkv, d, seed, pad_q=0, pad_k=0) -> PackedInputs:
    """Draw a packed bf16 batch: Q, K, V, dO in that order from ``seed``."""
    cu_q, cu_k = offsets(lens_q), offsets(lens_k)
    tq, tk = int(cu_q[-1]) + pad_q, int(cu_k[-1]) + pad_k
    rng = np.random.default_rng(seed)
    draws = [rng.standard_normal(s, dtype=np.float32) for s in ((tq, H, d), (tk, Hkv, d), (tk, Hkv, d), (tq, H, d))]
    bits = [bf16_bits(a) for a in draws]
    vals = [bf16_to_f32(b) for b in bits]
    return PackedInputs(list(lens_q), list(lens_k), H, Hkv, d, seed, cu_q, cu_k, *vals, *bits)


def length_mix(B: int, max_len: int, seed: int, min_len: int = 1) -> list:
    """B sequence lengths drawn uniformly from [min_len, max_len], one of them
    pinned to max_len so the batch reaches its stated maximum."""
    rng = np.random.default_rng(200 + seed)
    lens = rng.integers(min_len, max_len + 1, size=B).tolist()
    lens[int(rng.integers(0, B))] = max_len
    return lens


@dataclasses.dataclass(frozen=True)
class PackedWorkload:
    """A packed variable-length workload: B sequences whose key lengths are
    drawn by ``length_mix``, H query heads sharing Hkv K/V heads. Query
    lengths equal the key lengths, or are ``queries`` per sequence when that
    is set (decoding: a few new tokens against a long cache)."""
    name: str
    B: int
    max_len: int
    H: int
    Hkv: int
    d: int
    mask_kind: int
    backward: bool
    seed: int
    queries: int = 0

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    def lengths(self) -> list:
        return length_mix(self.B, self.max_len, self.seed, min_len=self.max_len // 8)

    def query_lengths(self) -> list:
        return [self.queries] * self.B if self.queries else self.lengths()


PACKED_WORKLOADS = {
    # 16 causal sequences of 512..4096 tokens packed back to back, 32 query
    # heads over 8 K/V heads (grouped-query attention), d = 128.
    "varlen_gqa": PackedWorkload("varlen_gqa", 16, 4096, 32, 8, 128, MASK_CAUSAL, True, 6),
    # decoding: one new query per sequence against 64 cached sequences of
    # 1024..8192 keys, 32 query heads over 8 K/V heads, d = 128.
    "decode_splitkv": PackedWorkload("decode_splitkv", 64, 8192, 32, 8, 128, MASK_CAUSAL, False, 7, queries=1),
}


# ---------------------------------------------------------------------------
# FP8 (OCP E4M3) codes: 1 sign, 4 exponent (bias 7), 3 mantissa bits; no
# infinities; S.1111.111 is NaN; largest finite 448, smallest subnormal 2^-9.
# ---------------------------------------------------------------------------
def fp8_e4m3_table() -> np.ndarray:
    """float32 value of each of the 256 E4M3 codes (NaN for 0x7F, 0xFF)."""
    codes = np.arange(256)
    s = np.where(codes & 0x80, -1.0, 1.0)
    e = (codes >> 3) & 15
    m = codes & 7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * 2.0 ** (e - 7.0))
    vals = (s * mag).astype(np.float32)
    vals[(e == 15) & (m == 7)] = np.nan
    return vals


_E4M3 = fp8_e4m3_table()
_E4M3_POS = _E4M3[:0x7F].astype(np.float64)      # codes 0x00..0x7E: 0 .. 448, increasing


def fp8_e4m3_bits(x: np.ndarray) -> np.ndarray:
    """float -> E4M3 codes (uint8), round to nearest, ties to the even code.
    Values beyond +-448 (and NaN) are rejected: callers scale into range."""
    x = np.asarray(x, dtype=np.float64)
    if not np.isfinite(x).all() or np.abs(x).max(initial=0.0) > 448.0:
        raise ValueError("E4M3 input out of range")
    a = np.abs(x)
    hi = np.clip(np.searchsorted(_E4M3_POS, a), 1, 0x7E)
    lo = hi - 1
    dlo, dhi = a - _E4M3_POS[lo], _E4M3_POS[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    return np.where(np.signbit(x), code | 0x80, code).astype(np.uint8)


def fp8_to_f32(bits: np.ndarray) -> np.ndarray:
    """E4M3 codes (uint8) -> their exact float32 values."""
    return _E4M3[np.asarray(bits, dtype=np.uint8)]


@dataclasses.dataclass
class Fp8Inputs:
    """FP8 inputs of one dense workload: codes q8, k8 [B, H, N, d] and
    vt8 [B, H, d, ldv] (V transposed, columns N..ldv-1 padding), their
    descale factors, and the dequantized fp32 values q, k, v [B, H, N, d]
    (exactly what the codes times the factors represent)."""
    q8: np.ndarray
    k8: np.ndarray
    vt8: np.ndarray
    ldv: int
    q_descale: float
    k_descale: float
    v_descale: float
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray


def fp8_inputs(B, H, N, d, seed, descale=2.0 ** -4, pad_code=0) -> Fp8Inputs:
    """Draw Q, K, V ~ N(0, 1) (seeded, in that order), quantize x / descale to
    E4M3 with one descale factor per tensor, and lay V out transposed with a
    leading dimension rounded up to 16 bytes (padding filled with pad_code)."""
    q, k, v = normal_tensors(seed, (B, H, N, d), 3)
    codes = [fp8_e4m3_bits(t / descale) for t in (q, k, v)]
    ldv = -(-N // 16) * 16
    vt8 = np.full((B, H, d, ldv), pad_code, dtype=np.uint8)
    vt8[..., :N] = np.swapaxes(codes[2], 2, 3)
    deq = [fp8_to_f32(c) * np.float32(descale) for c in codes]
    return Fp8Inputs(codes[0], codes[1], vt8, ldv, descale, descale, descale, *deq)


# FP8 forward workloads: the bf16 causal shapes with E4M3 inputs (per-tensor
# descale 2^-4), forward only.
FP8_WORKLOADS = {
    "causal_train_fp8": Workload("causal_train_fp8", 8, 16, 4096, 128, DTYPE_BF16, MASK_CAUSAL, False, 3),
    "long_prefill_fp8": Workload("long_prefill_fp8", 1, 32, 32768, 128, DTYPE_BF16, MASK_CAUSAL, False, 4),
}
