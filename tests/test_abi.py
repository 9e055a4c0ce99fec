"""The C-ABI library loads, exports what include/fa.h declares, and rejects
invalid arguments with the documented status before touching the GPU.

CPU only: every call below fails host-side validation, which runs before any
HIP API call, so no device is needed (pointers are fake, never dereferenced).
Where a GPU is visible the module is skipped: a regression in the host-side
validation must fail a test here, never launch a kernel on a fake address.
"""
import math
import os

import pytest
import torch

import io_aware_exact_10_amd as fa

pytestmark = pytest.mark.skipif(torch.cuda.is_available(),
                                reason="fake device pointers: host-validation tests run on the CPU build only")

A = 0x10000          # fake, 16-byte aligned "device" addresses
BIG = 1 << 30        # spacing so fake tensors never overlap


def ptrs(n):
    return [A + i * BIG for i in range(n)]


def fwd_args(**kw):
    q, k, v, o, lse = ptrs(5)
    args = dict(q=q, k=k, v=v, o=o, lse=lse, B=1, H=2, N=256, d=64, scale=0.125,
                mask_kind=fa.MASK_NONE, block_mask=None, dtype=fa.DTYPE_BF16, stream=None)
    args.update(kw)
    return args


def bwd_args(**kw):
    q, k, v, o, lse, do, dq, dk, dv, ws = ptrs(10)
    args = dict(q=q, k=k, v=v, o=o, lse=lse, dO=do, dq=dq, dk=dk, dv=dv, B=1, H=2, N=256, d=64,
                scale=0.125, mask_kind=fa.MASK_NONE, block_mask=None, dtype=fa.DTYPE_BF16,
                workspace=ws, workspace_bytes=fa.fa_bwd_workspace_bytes(1, 2, 256, 64), stream=None)
    args.update(kw)
    return args


def call_fwd(**kw):
    return fa.fa_fwd(**fwd_args(**kw))


def call_bwd(**kw):
    return fa.fa_bwd(**bwd_args(**kw))


def test_library_exports_every_declared_symbol():
    names = fa.declared_functions()
    assert set(names) == {"fa_fwd", "fa_fwd_tiled", "fa_bwd", "fa_bwd_rowterm", "fa_bwd_dkdv", "fa_bwd_dq",
                          "fa_bwd_workspace_bytes", "fa_status_string", "fa_fwd_varlen",
                          "fa_bwd_varlen", "fa_bwd_varlen_workspace_bytes", "fa_splitkv_splits",
                          "fa_splitkv_workspace_bytes", "fa_fwd_splitkv", "fa_fwd_fp8", "fa_bwd_noalloc",
                          "fa_debug_reverse_order"}
    L = fa.lib()
    for n in names:
        assert hasattr(L, n), n


def test_debug_reverse_order_switch():
    """The switch is host state only: it returns the previous setting."""
    prev = fa.fa_debug_reverse_order(1)
    assert prev in (0, 1)
    assert fa.fa_debug_reverse_order(7) == 1
    assert fa.fa_debug_reverse_order(0) == 1
    assert fa.fa_debug_reverse_order(prev) == 0
    assert fa.fa_debug_reverse_order(prev) == prev


def test_single_hip_runtime_in_process():
    """libfa.so must bind to the HIP runtime torch already loaded."""
    fa.lib()
    maps = open("/proc/self/maps").read().splitlines()
    hip = {line.split()[-1] for line in maps if "libamdhip64" in line}
    assert len(hip) == 1, hip


def test_status_strings():
    codes = [fa.FA_OK, fa.FA_ERR_NULL, fa.FA_ERR_SHAPE, fa.FA_ERR_UNSUPPORTED, fa.FA_ERR_MASK,
             fa.FA_ERR_WORKSPACE, fa.FA_ERR_ALIGN, fa.FA_ERR_HIP, fa.FA_ERR_ARG, fa.FA_ERR_SCRATCH]
    seen = set()
    for c in codes:
        s = fa.fa_status_string(c)
        assert s and s != "unknown status"
        seen.add(s)
    assert len(seen) == len(codes)
    assert fa.fa_status_string(-99) == "unknown status"


def test_workspace_bytes():
    """Two float arrays (row term, rescaled LSE), each rounded up to 256 bytes."""
    assert fa.fa_bwd_workspace_bytes(1, 1, 1, 64) == 2 * 256
    assert fa.fa_bwd_workspace_bytes(2, 3, 1000, 128) == 2 * ((2 * 3 * 1000 * 4 + 255) // 256) * 256
    assert fa.fa_bwd_workspace_bytes(64, 16, 1024, 64) == 2 * 64 * 16 * 1024 * 4
    for bad in ((0, 1, 1, 64), (1, 0, 1, 64), (1, 1, 0, 64), (1, 1, 8, 96)):
        assert fa.fa_bwd_workspace_bytes(*bad) == 0


@pytest.mark.parametrize("name", ["q", "k", "v", "o", "lse"])
def test_fwd_null(name):
    assert call_fwd(**{name: None}) == fa.FA_ERR_NULL


@pytest.mark.parametrize("name", ["q", "k", "v", "o", "lse", "dO", "dq", "dk", "dv"])
def test_bwd_null(name):
    assert call_bwd(**{name: None}) == fa.FA_ERR_NULL


@pytest.mark.parametrize("kw,code", [
    (dict(B=0), fa.FA_ERR_SHAPE), (dict(H=-1), fa.FA_ERR_SHAPE), (dict(N=0), fa.FA_ERR_SHAPE),
    (dict(B=1 << 20, H=1 << 20, N=1 << 10), fa.FA_ERR_SHAPE),
    (dict(d=32), fa.FA_ERR_UNSUPPORTED), (dict(d=96), fa.FA_ERR_UNSUPPORTED), (dict(d=256), fa.FA_ERR_UNSUPPORTED),
    (dict(dtype=2), fa.FA_ERR_UNSUPPORTED),
    (dict(mask_kind=3), fa.FA_ERR_MASK), (dict(mask_kind=-1), fa.FA_ERR_MASK),
    (dict(mask_kind=2, block_mask=None), fa.FA_ERR_MASK),
    (dict(scale=math.nan), fa.FA_ERR_ARG), (dict(scale=math.inf), fa.FA_ERR_ARG),
    (dict(q=A + 8), fa.FA_ERR_ALIGN), (dict(o=3 * BIG + A + 2), fa.FA_ERR_ALIGN),
    (dict(lse=4 * BIG + A + 2), fa.FA_ERR_ALIGN),
    (dict(o=A), fa.FA_ERR_ARG),                      # o aliases q
    (dict(lse=A + 64), fa.FA_ERR_ARG),               # lse inside q
])
def test_fwd_validation(kw, code):
    assert call_fwd(**kw) == code


def call_fwd_tiled(block_rows, **kw):
    return fa.fa_fwd_tiled(**fwd_args(**kw), block_rows=block_rows)


@pytest.mark.parametrize("block_rows,kw,code", [
    (16, {}, fa.FA_ERR_UNSUPPORTED), (96, {}, fa.FA_ERR_UNSUPPORTED), (512, {}, fa.FA_ERR_UNSUPPORTED),
    (-32, {}, fa.FA_ERR_UNSUPPORTED),
    (64, dict(dtype=fa.DTYPE_F32), fa.FA_ERR_UNSUPPORTED),          # chosen heights are bf16 only
    (256, dict(mask_kind=2, block_mask=A + 9 * BIG), fa.FA_ERR_UNSUPPORTED),   # straddles mask blocks
    (64, dict(q=None), fa.FA_ERR_NULL), (64, dict(N=0), fa.FA_ERR_SHAPE),
    (128, dict(d=96), fa.FA_ERR_UNSUPPORTED), (32, dict(mask_kind=5), fa.FA_ERR_MASK),
    (64, dict(q=A + 8), fa.FA_ERR_ALIGN), (64, dict(o=A), fa.FA_ERR_ARG),
    (0, dict(scale=math.nan), fa.FA_ERR_ARG),
])
def test_fwd_tiled_validation(block_rows, kw, code):
    """fa_fwd_tiled checks the tile height on top of fa_fwd's own checks."""
    assert call_fwd_tiled(block_rows, **kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(workspace=None), fa.FA_ERR_WORKSPACE),
    (dict(workspace_bytes=16), fa.FA_ERR_WORKSPACE),
    (dict(d=80), fa.FA_ERR_UNSUPPORTED),
    (dict(mask_kind=2, block_mask=None), fa.FA_ERR_MASK),
    (dict(scale=-math.inf), fa.FA_ERR_ARG),
    (dict(dq=6 * BIG + A + 4), fa.FA_ERR_ALIGN),
    (dict(workspace=9 * BIG + A + 8), fa.FA_ERR_ALIGN),
    (dict(dk=A + 2 * BIG), fa.FA_ERR_ARG),           # dk aliases v
    (dict(dv=6 * BIG + A), fa.FA_ERR_ARG),           # dv aliases dq
    (dict(workspace=8 * BIG + A + 128), fa.FA_ERR_ARG),  # workspace inside dv
])
def test_bwd_validation(kw, code):
    assert call_bwd(**kw) == code


def test_torch_wrappers_reject_bad_tensors():
    import torch
    q = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fa.forward(q, q, q)                           # CPU tensors
    with pytest.raises(ValueError):
        fa.forward(q[0], q[0], q[0])                  # wrong rank
    with pytest.raises(ValueError):
        fa.forward(q, q.float(), q)                   # mixed dtypes


def noalloc_args(**kw):
    a = bwd_args()
    del a["workspace"], a["workspace_bytes"]
    a.update(kw)
    return a


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), fa.FA_ERR_NULL),
    (dict(dv=None), fa.FA_ERR_NULL),
    (dict(N=0), fa.FA_ERR_SHAPE),
    (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(mask_kind=2, block_mask=None), fa.FA_ERR_MASK),
    (dict(scale=math.inf), fa.FA_ERR_ARG),
    (dict(dq=A + 8), fa.FA_ERR_ALIGN),
    (dict(dk=A + 2 * BIG), fa.FA_ERR_ARG),                         # dk aliases v
    # one row past the built-in scratch; the tensors (256 MiB each) still fit the fake 1 GiB spacing
    (dict(B=1, H=1, N=fa.FA_BWD_NOALLOC_MAX_ROWS + 1), fa.FA_ERR_SCRATCH),
    (dict(B=2, H=16, N=fa.FA_BWD_NOALLOC_MAX_ROWS // 32 + 64, d=64), fa.FA_ERR_SCRATCH),
])
def test_bwd_noalloc_validation(kw, code):
    """fa_bwd_noalloc validates like fa_bwd (no workspace arguments) and
    rejects problems past its built-in scratch before any HIP call."""
    assert fa.fa_bwd_noalloc(**noalloc_args(**kw)) == code


def test_torch_wrappers_reject_bad_outputs():
    """Caller-supplied outputs and workspaces are checked for shape, dtype and
    contiguity before anything is enqueued: the kernels write through raw
    pointers, so an undersized buffer would be written past its end."""
    bf = torch.bfloat16
    q = torch.zeros(2, 3, 8, 64, dtype=bf)
    lse = torch.zeros(2, 3, 8)
    with pytest.raises(ValueError, match="lse"):
        fa.forward(q, q, q, lse=torch.empty(1))
    with pytest.raises(ValueError, match="lse"):
        fa.forward(q, q, q, lse=torch.empty(2, 3, 8, dtype=bf))
    with pytest.raises(ValueError, match="out"):
        fa.forward(q, q, q, out=torch.empty(2, 3, 8, 32, dtype=bf))
    with pytest.raises(ValueError, match="out"):
        fa.forward(q, q, q, out=torch.empty(2, 3, 8, 64))                       # fp32 out for bf16 q
    with pytest.raises(ValueError, match="out"):
        fa.forward(q, q, q, out=torch.empty(2, 3, 64, 8, dtype=bf).transpose(2, 3))  # not contiguous
    with pytest.raises(ValueError, match="GPU"):
        fa.forward(q, q, q, out=torch.empty_like(q), lse=lse)                   # well formed, on the CPU
    for name in ("dq", "dk", "dv"):
        with pytest.raises(ValueError, match=name):
            fa.backward(q, q, q, q, lse, q, **{name: torch.empty(1, 3, 8, 64, dtype=bf)})
    with pytest.raises(ValueError, match="lse"):
        fa.backward(q, q, q, q, torch.zeros(2, 3, 7), q)
    with pytest.raises(ValueError, match="do"):
        fa.backward(q, q, q, q, lse, q[:, :, :4].contiguous())
    with pytest.raises(ValueError, match="workspace"):
        fa.backward(q, q, q, q, lse, q, workspace=torch.empty(8, dtype=torch.uint8))
    with pytest.raises(ValueError, match="GPU"):
        fa.backward(q, q, q, q, lse, q)
    # packed batches, split keys, FP8
    pq = torch.zeros(8, 4, 64, dtype=bf)
    pk = torch.zeros(8, 2, 64, dtype=bf)
    cu = torch.tensor([0, 8], dtype=torch.int32)
    with pytest.raises(ValueError, match="lse"):
        fa.forward_varlen(pq, pk, pk, cu, cu, 8, 8, lse=torch.empty(4, 7))
    with pytest.raises(ValueError, match="out"):
        fa.forward_varlen(pq, pk, pk, cu, cu, 8, 8, out=torch.empty_like(pk))
    plse = torch.zeros(4, 8)
    with pytest.raises(ValueError, match="dk"):
        fa.backward_varlen(pq, pk, pk, pq, plse, pq, cu, cu, 8, 8, dk=torch.empty_like(pq))
    with pytest.raises(ValueError, match="workspace"):
        fa.backward_varlen(pq, pk, pk, pq, plse, pq, cu, cu, 8, 8, workspace=torch.empty(4, dtype=torch.uint8))
    with pytest.raises(ValueError, match="lse"):
        fa.forward_splitkv(pq, pk, pk, cu, cu, 8, 8, lse=torch.empty(8, 4))
    with pytest.raises(ValueError, match="workspace"):
        fa.forward_splitkv(pq, pk, pk, cu, cu, 8, 8, workspace=torch.empty(4, dtype=torch.uint8))
    q8 = torch.zeros(1, 2, 16, 64, dtype=torch.uint8)
    vt8 = torch.zeros(1, 2, 64, 16, dtype=torch.uint8)
    with pytest.raises(ValueError, match="out"):
        fa.forward_fp8(q8, q8, vt8, out=torch.empty(1, 2, 16, 64))
    with pytest.raises(ValueError, match="lse"):
        fa.forward_fp8(q8, q8, vt8, lse=torch.empty(1, 2, 15))
    with pytest.raises(ValueError, match="GPU"):
        fa.forward_fp8(q8, q8, vt8)


def test_product_path_does_not_reference_the_oracle():
    """The package source must not import or call the CPU oracle."""
    pkg = os.path.dirname(fa.__file__)
    for root, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                txt = open(os.path.join(root, f)).read()
                assert "import oracle" not in txt and "from oracle" not in txt, f


def step_args(name, **kw):
    a = bwd_args()
    if name == "rowterm":
        keep = ["o", "dO", "lse", "B", "H", "N", "d", "dtype", "workspace", "workspace_bytes", "stream"]
    elif name == "dkdv":
        keep = ["q", "k", "v", "lse", "dO", "dk", "dv", "B", "H", "N", "d", "scale", "mask_kind",
                "block_mask", "dtype", "workspace", "workspace_bytes", "stream"]
    else:
        keep = ["q", "k", "v", "lse", "dO", "dq", "B", "H", "N", "d", "scale", "mask_kind",
                "block_mask", "dtype", "workspace", "workspace_bytes", "stream"]
    a = {k: a[k] for k in keep}
    a.update(kw)
    return a


STEPS = {"rowterm": fa.fa_bwd_rowterm, "dkdv": fa.fa_bwd_dkdv, "dq": fa.fa_bwd_dq}


@pytest.mark.parametrize("name", ["rowterm", "dkdv", "dq"])
def test_bwd_step_validation(name):
    f = STEPS[name]
    first = {"rowterm": "o", "dkdv": "q", "dq": "q"}[name]
    assert f(**step_args(name, **{first: None})) == fa.FA_ERR_NULL
    assert f(**step_args(name, d=96)) == fa.FA_ERR_UNSUPPORTED
    assert f(**step_args(name, N=0)) == fa.FA_ERR_SHAPE
    assert f(**step_args(name, workspace=None)) == fa.FA_ERR_WORKSPACE
    assert f(**step_args(name, workspace_bytes=8)) == fa.FA_ERR_WORKSPACE
    assert f(**step_args(name, workspace=9 * BIG + A + 4)) == fa.FA_ERR_ALIGN
    if name != "rowterm":
        assert f(**step_args(name, mask_kind=2, block_mask=None)) == fa.FA_ERR_MASK
        assert f(**step_args(name, scale=math.nan)) == fa.FA_ERR_ARG
        out = "dk" if name == "dkdv" else "dq"
        assert f(**step_args(name, **{out: A})) == fa.FA_ERR_ARG          # output aliases q
        assert f(**step_args(name, lse=4 * BIG + A + 1)) == fa.FA_ERR_ALIGN
    else:
        assert f(**step_args(name, workspace=A + 3 * BIG)) == fa.FA_ERR_ARG   # workspace aliases o
        assert f(**step_args(name, lse=None)) == fa.FA_ERR_NULL
        assert f(**step_args(name, workspace=A + 4 * BIG)) == fa.FA_ERR_ARG   # workspace aliases lse


# --------------------------------------------------------------------------
# packed variable-length calls
# --------------------------------------------------------------------------
def vfwd_args(**kw):
    q, k, v, o, lse, cq, ck = ptrs(7)
    args = dict(q=q, k=k, v=v, o=o, lse=lse, cu_seqlens_q=cq, cu_seqlens_k=ck, B=2, H=4, Hkv=2,
                max_seqlen_q=100, max_seqlen_k=120, total_q=150, total_k=200, d=64, scale=0.125,
                mask_kind=fa.MASK_CAUSAL, dtype=fa.DTYPE_BF16, stream=None)
    args.update(kw)
    return args


def vbwd_args(**kw):
    q, k, v, o, lse, do, dq, dk, dv, cq, ck, ws = ptrs(12)
    args = dict(q=q, k=k, v=v, o=o, lse=lse, dO=do, dq=dq, dk=dk, dv=dv, cu_seqlens_q=cq, cu_seqlens_k=ck,
                B=2, H=4, Hkv=2, max_seqlen_q=100, max_seqlen_k=120, total_q=150, total_k=200, d=64,
                scale=0.125, mask_kind=fa.MASK_NONE, dtype=fa.DTYPE_BF16, workspace=ws,
                workspace_bytes=fa.fa_bwd_varlen_workspace_bytes(150, 4, 64), stream=None)
    args.update(kw)
    return args


def test_varlen_workspace_bytes():
    assert fa.fa_bwd_varlen_workspace_bytes(150, 4, 64) == 2 * 2560
    assert fa.fa_bwd_varlen_workspace_bytes(1, 1, 128) == 2 * 256
    for bad in ((0, 1, 64), (1, 0, 64), (5, 2, 32)):
        assert fa.fa_bwd_varlen_workspace_bytes(*bad) == 0


@pytest.mark.parametrize("name", ["q", "k", "v", "o", "lse", "cu_seqlens_q", "cu_seqlens_k"])
def test_varlen_fwd_null(name):
    assert fa.fa_fwd_varlen(**vfwd_args(**{name: None})) == fa.FA_ERR_NULL


@pytest.mark.parametrize("kw,code", [
    (dict(B=0), fa.FA_ERR_SHAPE), (dict(H=0), fa.FA_ERR_SHAPE), (dict(Hkv=0), fa.FA_ERR_SHAPE),
    (dict(H=6, Hkv=4), fa.FA_ERR_SHAPE), (dict(H=1 << 17, Hkv=1), fa.FA_ERR_SHAPE),
    (dict(max_seqlen_q=0), fa.FA_ERR_SHAPE), (dict(max_seqlen_k=0), fa.FA_ERR_SHAPE),
    (dict(total_q=0), fa.FA_ERR_SHAPE), (dict(total_k=-3), fa.FA_ERR_SHAPE),
    (dict(total_q=1 << 30, H=1 << 12, Hkv=1), fa.FA_ERR_SHAPE),
    (dict(d=96), fa.FA_ERR_UNSUPPORTED), (dict(dtype=fa.DTYPE_F32), fa.FA_ERR_UNSUPPORTED),
    (dict(mask_kind=fa.MASK_BLOCK_SPARSE), fa.FA_ERR_MASK), (dict(mask_kind=7), fa.FA_ERR_MASK),
    (dict(scale=math.nan), fa.FA_ERR_ARG),
    (dict(q=A + 4), fa.FA_ERR_ALIGN), (dict(cu_seqlens_k=6 * BIG + A + 2), fa.FA_ERR_ALIGN),
    (dict(o=A + 2 * BIG), fa.FA_ERR_ARG),            # o aliases v
    (dict(lse=5 * BIG + A), fa.FA_ERR_ARG),          # lse aliases cu_seqlens_q
])
def test_varlen_fwd_validation(kw, code):
    assert fa.fa_fwd_varlen(**vfwd_args(**kw)) == code


@pytest.mark.parametrize("kw,code", [
    (dict(dv=None), fa.FA_ERR_NULL), (dict(cu_seqlens_q=None), fa.FA_ERR_NULL),
    (dict(H=3, Hkv=2), fa.FA_ERR_SHAPE), (dict(dtype=fa.DTYPE_F32), fa.FA_ERR_UNSUPPORTED),
    (dict(mask_kind=fa.MASK_BLOCK_SPARSE), fa.FA_ERR_MASK),
    (dict(workspace=None), fa.FA_ERR_WORKSPACE), (dict(workspace_bytes=100), fa.FA_ERR_WORKSPACE),
    (dict(dk=7 * BIG + A + 8), fa.FA_ERR_ALIGN), (dict(workspace=11 * BIG + A + 4), fa.FA_ERR_ALIGN),
    (dict(dq=A), fa.FA_ERR_ARG),                     # dq aliases q
    (dict(dv=7 * BIG + A), fa.FA_ERR_ARG),           # dv aliases dk
    (dict(workspace=9 * BIG + A), fa.FA_ERR_ARG),    # workspace aliases cu_seqlens_q
])
def test_varlen_bwd_validation(kw, code):
    assert fa.fa_bwd_varlen(**vbwd_args(**kw)) == code


def test_varlen_torch_wrappers_reject_bad_tensors():
    import torch
    q = torch.zeros(8, 2, 64, dtype=torch.bfloat16)
    cu = torch.tensor([0, 8], dtype=torch.int32)
    with pytest.raises(ValueError):
        fa.forward_varlen(q, q, q, cu, cu, 8, 8)          # CPU tensors
    with pytest.raises(ValueError):
        fa.forward_varlen(q[None], q, q, cu, cu, 8, 8)    # wrong rank


# --------------------------------------------------------------------------
# split-key forward
# --------------------------------------------------------------------------
def skv_args(**kw):
    q, k, v, o, lse, cq, ck, ws = ptrs(8)
    args = dict(q=q, k=k, v=v, o=o, lse=lse, cu_seqlens_q=cq, cu_seqlens_k=ck, B=4, H=32, Hkv=8,
                max_seqlen_q=2, max_seqlen_k=5000, total_q=8, total_k=20000, d=128, scale=0.088,
                mask_kind=fa.MASK_CAUSAL, dtype=fa.DTYPE_BF16, num_splits=0, workspace=ws,
                workspace_bytes=1 << 24, stream=None)
    args.update(kw)
    return args


def test_splitkv_split_choice_and_workspace():
    assert fa.fa_splitkv_splits(4, 8, 5000, 0) == 20          # ceil(5000 / 256): ranges of >= 256 keys
    assert fa.fa_splitkv_splits(64, 8, 100000, 0) == 16       # 512 (sequence, head) groups x 16 = 8192
    assert fa.fa_splitkv_splits(1, 1, 64, 0) == 1
    assert fa.fa_splitkv_splits(1, 1, 1 << 20, 0) == 128      # capped
    assert fa.fa_splitkv_splits(2, 2, 100, 7) == 7            # forced
    assert fa.fa_splitkv_splits(2, 2, 100, 129) == fa.FA_ERR_ARG
    assert fa.fa_splitkv_splits(2, 2, 100, -1) == fa.FA_ERR_ARG
    assert fa.fa_splitkv_splits(0, 2, 100, 0) == fa.FA_ERR_SHAPE
    assert fa.fa_splitkv_workspace_bytes(8, 32, 128, 20) == 20 * 8 * 32 * 128 * 4 + 20 * 32 * 8 * 4
    assert fa.fa_splitkv_workspace_bytes(8, 32, 128, 0) == 0
    assert fa.fa_splitkv_workspace_bytes(8, 32, 96, 1) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), fa.FA_ERR_NULL), (dict(cu_seqlens_k=None), fa.FA_ERR_NULL),
    (dict(H=6, Hkv=4), fa.FA_ERR_SHAPE), (dict(max_seqlen_q=0), fa.FA_ERR_SHAPE),
    (dict(max_seqlen_q=17, H=32, Hkv=4), fa.FA_ERR_UNSUPPORTED),     # 8 x 17 > 128 stacked rows
    (dict(d=256), fa.FA_ERR_UNSUPPORTED), (dict(dtype=fa.DTYPE_F32), fa.FA_ERR_UNSUPPORTED),
    (dict(mask_kind=fa.MASK_BLOCK_SPARSE), fa.FA_ERR_MASK), (dict(scale=math.inf), fa.FA_ERR_ARG),
    (dict(num_splits=200), fa.FA_ERR_ARG),
    (dict(workspace=None), fa.FA_ERR_WORKSPACE), (dict(workspace_bytes=1024), fa.FA_ERR_WORKSPACE),
    (dict(workspace=7 * BIG + A + 8), fa.FA_ERR_ALIGN), (dict(lse=4 * BIG + A + 2), fa.FA_ERR_ALIGN),
    (dict(o=A + BIG), fa.FA_ERR_ARG),                 # o aliases k
    (dict(workspace=5 * BIG + A), fa.FA_ERR_ARG),     # workspace aliases cu_seqlens_q
])
def test_splitkv_validation(kw, code):
    assert fa.fa_fwd_splitkv(**skv_args(**kw)) == code


# --------------------------------------------------------------------------
# FP8 forward
# --------------------------------------------------------------------------
def f8_args(**kw):
    q, k, vt, o, lse = ptrs(5)
    args = dict(q=q, k=k, v_t=vt, o=o, lse=lse, B=1, H=2, N=100, d=128, ldv=112, scale=0.088,
                q_descale=0.0625, k_descale=0.0625, v_descale=0.0625, mask_kind=fa.MASK_CAUSAL, stream=None)
    args.update(kw)
    return args


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), fa.FA_ERR_NULL), (dict(v_t=None), fa.FA_ERR_NULL), (dict(lse=None), fa.FA_ERR_NULL),
    (dict(N=0), fa.FA_ERR_SHAPE), (dict(ldv=96), fa.FA_ERR_SHAPE), (dict(ldv=120), fa.FA_ERR_SHAPE),
    (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(mask_kind=fa.MASK_BLOCK_SPARSE), fa.FA_ERR_MASK), (dict(mask_kind=5), fa.FA_ERR_MASK),
    (dict(scale=math.nan), fa.FA_ERR_ARG), (dict(v_descale=math.inf), fa.FA_ERR_ARG),
    (dict(q_descale=1e30, k_descale=1e30), fa.FA_ERR_ARG),        # product overflows
    (dict(k=BIG + A + 8), fa.FA_ERR_ALIGN), (dict(lse=4 * BIG + A + 1), fa.FA_ERR_ALIGN),
    (dict(o=A + 2 * BIG), fa.FA_ERR_ARG),                           # o aliases v_t
])
def test_fp8_validation(kw, code):
    assert fa.fa_fwd_fp8(**f8_args(**kw)) == code
