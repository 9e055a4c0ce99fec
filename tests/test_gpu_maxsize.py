"""A tensor of more than 2^31 elements: B = 1, H = 64, N = 2^18 + 64, d = 128
(2 164 260 864 elements, 4.3 GB per bf16 tensor), causal, forward and
backward through the C ABI. Every index past 2^31 must be formed in 64-bit
arithmetic. The oracle checks the last 512 positions of the last head, all of
which lie past element 2^31: under the causal mask those keys are seen only by
those queries, so the sub-problem "the last 512 queries against all keys"
(bottom-right aligned) gives their exact dQ, dK and dV rows, and the forward
rows.

Inputs are drawn on the device by torch's seeded generator (N(0, 1), rounded
to bf16) and copied to the host for the oracle; nothing the oracle sees comes
from the HIP path.
"""
import math

import numpy as np
import pytest
import torch

import io_aware_exact_10_amd as fa
import oracle
import synth
from gpu_util import announce, check_forward, check_grad

pytestmark = pytest.mark.gpu

B, H, N, D = 1, 64, (1 << 18) + 64, 128
TAIL = 512


def test_more_than_2_pow_31_elements_causal():
    assert B * H * N * D > 2 ** 31
    assert (H - 1) * N * D + (N - TAIL) * D >= 2 ** 31   # the checked rows lie past element 2^31
    gen = torch.Generator(device="cuda")
    gen.manual_seed(20260)
    t = {}
    for name in ("q", "k", "v", "do"):
        x = torch.randn((B, H, N, D), generator=gen, device="cuda", dtype=torch.float32)
        t[name] = x.to(torch.bfloat16)
        del x
    torch.cuda.synchronize()
    scale = 1.0 / math.sqrt(D)
    announce(f"fa_fwd max size B{B} H{H} N{N} d{D} causal")
    o, lse = fa.forward(t["q"], t["k"], t["v"], scale, synth.MASK_CAUSAL)
    announce("fa_bwd max size")
    dq, dk, dv = fa.backward(t["q"], t["k"], t["v"], o, lse, t["do"], scale, synth.MASK_CAUSAL)
    torch.cuda.synchronize()

    h = H - 1
    host = {n: t[n][0, h].float().cpu().numpy().astype(np.float64) for n in t}
    got = dict(o=o[0, h, N - TAIL:].float().cpu().numpy(), lse=lse[0, h, N - TAIL:].cpu().numpy(),
               dq=dq[0, h, N - TAIL:].float().cpu().numpy(), dk=dk[0, h, N - TAIL:].float().cpu().numpy(),
               dv=dv[0, h, N - TAIL:].float().cpu().numpy())
    del t, o, lse, dq, dk, dv
    torch.cuda.empty_cache()

    q_tail, do_tail = host["q"][N - TAIL:], host["do"][N - TAIL:]
    O, L = oracle.forward_head(q_tail, host["k"], host["v"], scale, synth.MASK_CAUSAL, chunk=128)
    check_forward(got["o"], got["lse"], O, L, synth.DTYPE_BF16, "max size, last head, last rows")
    gq, gk, gv = oracle.backward_head(q_tail, host["k"], host["v"], do_tail, scale, synth.MASK_CAUSAL, chunk=128)
    check_grad(got["dq"], gq, synth.DTYPE_BF16, "max size dq")
    check_grad(got["dk"], gk[N - TAIL:], synth.DTYPE_BF16, "max size dk")
    check_grad(got["dv"], gv[N - TAIL:], synth.DTYPE_BF16, "max size dv")
