"""Helpers shared by the GPU parity tests: seeded inputs to device tensors,
one call of the HIP path through the C ABI, and the comparison metrics.

Tolerances (written here, used by every GPU test):
  bf16 inputs: max |dO| <= 2e-2 on O, max |dLSE| <= 1e-3 on LSE; gradients
  max |dg| / max |g_ref| <= 5e-2 per tensor against the oracle run on the
  bf16-rounded inputs. fp32 inputs: max |dO| <= 1e-4, max |dLSE| <= 1e-4,
  gradients max-normalised <= 1e-4.
The normaliser of the gradient check is max(max |g_ref|, 1e-3): where the
exact gradient vanishes (a single visible key makes dQ identically 0) the
bound becomes absolute, 1e-3 x the tolerance.
Besides the max-normalised bound the gradient checks also bound the relative
Frobenius error (bf16 2e-2, fp32 1e-4): rounding P and dS to bf16 costs
about 2^-9 per element, i.e. a few 1e-3 in Frobenius norm, so a larger value
means a real defect even when the max-normalised bound still passes.
"""
import sys

import numpy as np
import torch

import io_aware_exact_10_amd as fa
import synth

O_TOL = {synth.DTYPE_BF16: 2e-2, synth.DTYPE_F32: 1e-4}
LSE_TOL = {synth.DTYPE_BF16: 1e-3, synth.DTYPE_F32: 1e-4}
GRAD_TOL = {synth.DTYPE_BF16: 5e-2, synth.DTYPE_F32: 1e-4}
GRAD_FRO_TOL = {synth.DTYPE_BF16: 2e-2, synth.DTYPE_F32: 1e-4}
GRAD_FLOOR = 1e-3


def announce(msg: str) -> None:
    """Name the case on stderr (bypassing pytest capture) before a GPU step."""
    sys.__stderr__.write(f"[gpu] {msg}\n")
    sys.__stderr__.flush()


def dev_tensor(vals: np.ndarray, bits, dtype: int) -> torch.Tensor:
    if dtype == synth.DTYPE_BF16:
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(vals, dtype=np.float32)).cuda()


def to_device(inp: synth.Inputs):
    w = inp.w
    t = dict(q=dev_tensor(inp.q, inp.q_bits, w.dtype), k=dev_tensor(inp.k, inp.k_bits, w.dtype),
             v=dev_tensor(inp.v, inp.v_bits, w.dtype))
    if inp.do is not None:
        t["do"] = dev_tensor(inp.do, inp.do_bits, w.dtype)
    t["mask"] = torch.from_numpy(inp.mask).cuda() if inp.mask is not None else None
    return t


def run_hip(inp: synth.Inputs, backward: bool, scale=None, mask_override=None):
    """Forward (and backward) through libfa; returns float64 numpy arrays."""
    w = inp.w
    scale = w.scale if scale is None else scale
    t = to_device(inp)
    mask = t["mask"] if mask_override is None else mask_override
    announce(f"fa_fwd {w.name} B{w.B} H{w.H} N{w.N} d{w.d} dtype{w.dtype} mask{w.mask_kind} scale{scale:.4g} seed{w.seed}")
    o, lse = fa.forward(t["q"], t["k"], t["v"], scale, w.mask_kind, mask)
    torch.cuda.synchronize()
    out = dict(o=o.float().cpu().numpy().astype(np.float64), lse=lse.cpu().numpy().astype(np.float64))
    if backward:
        announce(f"fa_bwd {w.name}")
        dq, dk, dv = fa.backward(t["q"], t["k"], t["v"], o, lse, t["do"], scale, w.mask_kind, mask)
        torch.cuda.synchronize()
        for n, x in (("dq", dq), ("dk", dk), ("dv", dv)):
            out[n] = x.float().cpu().numpy().astype(np.float64)
    return out


def max_abs(a, b):
    """max |a - b| treating matching infinities (e.g. empty-row LSE) as equal."""
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    same_inf = np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))
    with np.errstate(invalid="ignore"):
        d = np.where(same_inf, 0.0, np.abs(a - b))
    return float(np.nan_to_num(d, nan=np.inf).max()) if d.size else 0.0


def check_forward(got_o, got_lse, ref_o, ref_lse, dtype, what=""):
    eo = max_abs(got_o, ref_o)
    el = max_abs(got_lse, ref_lse)
    assert eo <= O_TOL[dtype], f"{what}: max|dO| = {eo:.3g} > {O_TOL[dtype]}"
    assert el <= LSE_TOL[dtype], f"{what}: max|dLSE| = {el:.3g} > {LSE_TOL[dtype]}"
    return eo, el


def check_grad(got, ref, dtype, what=""):
    ref = np.asarray(ref, np.float64)
    got = np.asarray(got, np.float64)
    scale = max(float(np.abs(ref).max()), GRAD_FLOOR)
    e = float(np.abs(got - ref).max()) / scale
    fro = float(np.linalg.norm(got - ref) / max(float(np.linalg.norm(ref)), GRAD_FLOOR * np.sqrt(ref.size)))
    assert np.isfinite(got).all(), f"{what}: non-finite gradient"
    assert e <= GRAD_TOL[dtype], f"{what}: max-normalised error {e:.3g} > {GRAD_TOL[dtype]}"
    assert fro <= GRAD_FRO_TOL[dtype], f"{what}: relative Frobenius error {fro:.3g} > {GRAD_FRO_TOL[dtype]}"
    return e, fro
