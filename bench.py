#!/usr/bin/env python3
"""Benchmark of the exact tiled attention hot path on one MI355X.

A step is one pass of the whole path over one batch of synthetic input:
fa_fwd (O and LSE), followed by fa_bwd (row term, dK/dV, dQ) where the
workload has a backward pass, through the C ABI. The default workload is the
largest one, the long-context causal prefill (B=1, H=32, N=32768, d=128,
bf16, forward only); ``--workload`` selects any other. Inputs are resident in
device memory before the timed region starts. ``value`` is the mean over the
timed steps; the median and the minimum are reported beside it.

Prints ONE JSON line (rank 0) with the metric in TFLOP/s under the FLOP
convention fwd = 4*d*vis, bwd = 10*d*vis per head (vis = visible
query/key pairs), plus:
  kernels       each kernel's mean duration per step from HIP events on the
                launch stream (the backward is enqueued as its three steps,
                fa_bwd_rowterm, fa_bwd_dkdv and fa_bwd_dq, the exact work
                fa_bwd does) and its algorithmic FLOPs per launch: fwd
                4*d*vis, dK/dV 8*d*vis (S, dP, dV, dK), dQ 2*d*vis (its S
                and dP are recomputation and not counted);
  roofline      the dominant (longest) kernel's achieved TFLOP/s against the
                MI355X dense bf16 MFMA peak, with its HBM traffic per launch
                from rocprofv3 FETCH_SIZE + WRITE_SIZE (profiles/traffic.json)
                when those counters were taken on the current source;
  cpu_baseline  the float64 CPU oracle timed on a bounded sample of the same
                workload on this host's cores;
  naive         the materialise-S torch composition (matmul, mask, softmax,
                matmul, autograd) on the same inputs, for comparison;
  also          (forward-only workloads) the forward + backward step of the
                causal training shape (B=8, H=16, N=4096, d=128), timed the
                same way on device-drawn inputs.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402

PEAK_BF16_TFLOPS = 256 * 2.4e9 * 4096 / 1e12     # 2516.6: 256 CUs x 2.4 GHz x 4096 FLOP/clk
PEAK_F32_VALU_TFLOPS = 157.3
PEAK_FP8_TFLOPS = 256 * 2.4e9 * 8192 / 1e12      # 5033.2: the published dense FP8 MFMA peak (5.0 PFLOP/s)
A100_FIG2_MS = 7.3                                # the pages' GPT-2-medium attention runtime (context)
PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_NAMES = {"fwd": "fwd_bf16_kernel", "rowterm": "bwd_rowterm_bf16_kernel",
                "dkdv": "bwd_dkdv_bf16_kernel", "dq": "bwd_dq_bf16_kernel",
                "splitkv": "splitkv_bf16_kernel", "combine": "splitkv_combine_kernel", "fwd_fp8": "fwd_fp8_kernel"}
_CSRC = "io_aware_exact_10_amd/csrc/"
KERNEL_SOURCES = {"fwd": (_CSRC + "fa_fwd_bf16.hip", _CSRC + "fa_common.h"),
                  "rowterm": (_CSRC + "fa_bwd_bf16.hip", _CSRC + "fa_common.h"),
                  "dkdv": (_CSRC + "fa_bwd_bf16.hip", _CSRC + "fa_common.h"),
                  "dq": (_CSRC + "fa_bwd_bf16.hip", _CSRC + "fa_common.h"),
                  "splitkv": (_CSRC + "fa_splitkv_bf16.hip", _CSRC + "fa_common.h"),
                  "combine": (_CSRC + "fa_splitkv_bf16.hip", _CSRC + "fa_common.h"),
                  "fwd_fp8": (_CSRC + "fa_fwd_fp8.hip", _CSRC + "fa_common.h")}


def measured_traffic(workload: str, key: str):
    """HBM bytes per launch of kernel `key` on `workload` from the committed
    counter summary, or None when absent or taken on other kernel source."""
    if not os.path.exists(PROFILE_TRAFFIC):
        return None
    rec = json.load(open(PROFILE_TRAFFIC)).get(workload, {}).get(key)
    if rec and rec.get("source_digest") == source_digest(*KERNEL_SOURCES[key]):
        return rec.get("hbm_bytes_per_launch")
    return None


def hbm_rate(traffic, ms):
    """Achieved HBM GB/s of a launch: measured bytes per launch over its mean
    duration (None when the bytes are not measured for this kernel source)."""
    return None if traffic is None or not ms else round(traffic / (ms * 1e-3) / 1e9, 1)


def copy_calibration(nbytes: int, dev) -> None:
    """One device-to-device copy of nbytes: the reference dispatch the
    FETCH_SIZE / WRITE_SIZE counters are scaled by."""
    if not nbytes:
        return
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def visible_pairs(w: synth.Workload, mask: np.ndarray | None) -> int:
    """Visible (query, key) pairs per head."""
    N = w.N
    if w.mask_kind == synth.MASK_NONE:
        return N * N
    if w.mask_kind == synth.MASK_CAUSAL:
        return N * (N + 1) // 2
    nb = mask.shape[0]
    sizes = np.array([min(128, N - 128 * i) for i in range(nb)], dtype=np.int64)
    return int((mask.astype(np.int64) * np.outer(sizes, sizes)).sum())


def source_digest(*files: str) -> str:
    """Digest of the kernel sources with comments and blank space removed,
    so that a counter record stays valid across comment-only edits and goes
    stale on any change of the code itself."""
    h = hashlib.sha256()
    for f in files:
        src = open(os.path.join(ROOT, f)).read()
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
        src = re.sub(r"//[^\n]*", " ", src)
        h.update(" ".join(src.split()).encode())
    return h.hexdigest()[:16]


def visible_pairs_rows(w: synth.Workload, mask: np.ndarray | None, rows: np.ndarray) -> int:
    """Visible (query, key) pairs of the query ``rows`` of one head."""
    rows = np.asarray(rows, dtype=np.int64)
    if w.mask_kind == synth.MASK_NONE:
        return int(rows.size) * w.N
    if w.mask_kind == synth.MASK_CAUSAL:
        return int(np.minimum(rows + 1, w.N).sum())
    nb = mask.shape[0]
    sizes = np.array([min(128, w.N - 128 * i) for i in range(nb)], dtype=np.int64)
    return int((mask[rows // 128].astype(np.int64) * sizes[None, :]).sum())


CPU_SAMPLE_ROWS = 2048   # query rows per head the oracle takes for sequences longer than 8K


def cpu_baseline(inp: synth.Inputs, budget_s: float, backward: bool, flop_per_head: float) -> dict:
    """Times the float64 oracle (as it stands) on whole heads until ~budget_s.

    For sequences longer than 8K the oracle takes every (N / 2048)-th query
    row of each head (forward only; the rows spread over the whole causal
    triangle) and is credited with the algorithmic FLOPs of exactly those
    rows, 4 * d per visible pair."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([t.get("num_threads", 1) for t in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        threads = len(os.sched_getaffinity(0))
    w = inp.w
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    rows = None
    if w.N > 8192:
        rows = np.arange(0, w.N, w.N // CPU_SAMPLE_ROWS)
        row_flop = 4.0 * w.d * visible_pairs_rows(w, inp.mask, rows)
    done = 0
    flops = 0.0
    t0 = time.perf_counter()
    for b, h in heads:
        oracle.forward_head(inp.q[b, h], inp.k[b, h], inp.v[b, h], w.scale, w.mask_kind, inp.mask, rows)
        if backward and rows is None:
            oracle.backward_head(inp.q[b, h], inp.k[b, h], inp.v[b, h], inp.do[b, h], w.scale, w.mask_kind, inp.mask)
        done += 1
        flops += flop_per_head if rows is None else row_flop
        if time.perf_counter() - t0 > budget_s:
            break
    el = time.perf_counter() - t0
    what = "fwd+bwd" if backward and rows is None else "fwd"
    sample = f"{done} of {len(heads)} heads, {what}" + (
        f", every {w.N // CPU_SAMPLE_ROWS}th query row ({rows.size} rows per head)" if rows is not None else "")
    return {"value": flops / el / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": sample, "seconds": round(el, 2)}


def naive_step(q, k, v, do, scale, mask_kind, bool_mask, backward):
    """Materialise-S comparator: S and P go through device memory.

    Returns O and, with ``backward``, the gradients (dQ, dK, dV) autograd
    gives for the upstream gradient ``do`` (else None)."""
    import torch
    qq = q.detach().requires_grad_(backward)
    kk = k.detach().requires_grad_(backward)
    vv = v.detach().requires_grad_(backward)
    s = torch.matmul(qq, kk.transpose(-1, -2).contiguous()) * scale
    if bool_mask is not None:
        s = s.masked_fill(~bool_mask, float("-inf"))
    p = torch.softmax(s.float(), dim=-1).to(q.dtype)
    o = torch.matmul(p, vv)
    if backward:
        o.backward(do)
        return o.detach(), (qq.grad, kk.grad, vv.grad)
    return o.detach(), None


NAIVE_WHOLE_N = 4096   # longer sequences run the comparator one head at a time (S, P of one head: N^2 elements)


def naive_mask(w, mask_t, dev):
    import torch
    if w.mask_kind == synth.MASK_CAUSAL:
        return torch.ones(w.N, w.N, dtype=torch.bool, device=dev).tril()
    if w.mask_kind == synth.MASK_BLOCK_SPARSE:
        return mask_t.bool().repeat_interleave(128, 0).repeat_interleave(128, 1)[: w.N, : w.N]
    return None


def naive_full(q, k, v, do, scale, mask_kind, bool_mask, backward):
    """The comparator over the whole batch, or head by head for long sequences."""
    if q.shape[2] <= NAIVE_WHOLE_N:
        return naive_step(q, k, v, do, scale, mask_kind, bool_mask, backward)
    for b in range(q.shape[0]):
        for h in range(q.shape[1]):
            sl = (slice(b, b + 1), slice(h, h + 1))
            naive_step(q[sl], k[sl], v[sl], do[sl] if backward else None, scale, mask_kind, bool_mask, backward)
    return None


# ---------------------------------------------------------------------------
# rocprofv3 summaries (text for profiles/), read from the SQLite output
# ---------------------------------------------------------------------------
KEYS_BY_SUBSTR = (("fwd_bf16_kernel", "fwd"), ("bwd_rowterm_bf16_kernel", "rowterm"),
                  ("bwd_dkdv_bf16_kernel", "dkdv"), ("bwd_dkdv8_bf16_kernel", "dkdv"), ("bwd_dq_bf16_kernel", "dq"),
                  ("splitkv_bf16_kernel", "splitkv"), ("splitkv_combine_kernel", "combine"),
                  ("fwd_fp8_kernel", "fwd_fp8"))
COPY_KERNEL = "__amd_rocclr_copyBuffer"


def summarize_trace(db_path: str) -> str:
    import sqlite3
    cur = sqlite3.connect(db_path).cursor()
    rows = cur.execute("select name, total_calls, average, percentage from top_kernels").fetchall()
    out = ["| kernel | calls | mean duration (us) | share of GPU time (%) |", "|---|---|---|---|"]
    for name, calls, avg, pct in rows:
        out.append(f"| `{name}` | {calls} | {avg:.2f} | {pct:.1f} |")
    return "\n".join(out)


def _pmc_means(db_path: str, counter: str) -> dict:
    """Mean counter value per dispatch of each kernel. For the copy kernel the
    largest dispatch is taken: the calibration copy is the biggest one (input
    uploads can run small copies through the same kernel)."""
    import collections
    import sqlite3
    cur = sqlite3.connect(db_path).cursor()
    per = collections.defaultdict(lambda: collections.defaultdict(float))
    for name, did, val in cur.execute(
            "select kernel_name, dispatch_id, value from counters_collection where counter_name = ?", (counter,)):
        per[name][did] += val
    out = {}
    for n, d in per.items():
        out[n] = max(d.values()) if COPY_KERNEL in n else sum(d.values()) / len(d)
    return out


COUNTER_SET = ("GRBM_GUI_ACTIVE", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_VALU_MFMA_MOPS_BF16",
               "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS", "SQ_LDS_BANK_CONFLICT", "SQ_INSTS_VALU_TRANS_F32",
               "SQ_WAVE_CYCLES")
N_XCD, N_SIMD = 8, 1024


def summarize_counters(db_path: str, substrs=("fa::",)) -> str:
    """Per-kernel means over dispatches of the COUNTER_SET pass, with three
    derived figures: the shader clock (GRBM_GUI_ACTIVE is summed over the 8
    XCDs; divided by the dispatch's duration in the same run), the MFMA busy
    fraction (SQ_VALU_MFMA_BUSY_CYCLES is per SIMD, 1024 SIMDs) and the
    executed MFMA work (SQ_INSTS_VALU_MFMA_MOPS_BF16 counts units of 512 FLOPs)."""
    import collections
    import sqlite3
    cur = sqlite3.connect(db_path).cursor()
    vals = collections.defaultdict(lambda: collections.defaultdict(lambda: collections.defaultdict(float)))
    dur = collections.defaultdict(dict)
    for name, did, cn, v, d in cur.execute(
            "select kernel_name, dispatch_id, counter_name, value, duration from counters_collection"):
        vals[name][cn][did] += v
        dur[name][did] = d
    lines = ["| kernel | dispatches | mean ns | clock GHz | MFMA busy | executed MFMA GFLOP | "
             + " | ".join(COUNTER_SET) + " |", "|" + "---|" * (6 + len(COUNTER_SET))]
    for name in sorted(vals):
        if not any(s in name for s in substrs):
            continue
        c = {cn: sum(d.values()) / len(d) for cn, d in vals[name].items()}
        ns = sum(dur[name].values()) / len(dur[name])
        cyc = c.get("GRBM_GUI_ACTIVE", 0.0) / N_XCD
        ghz = cyc / ns if ns else 0.0
        busy = c.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / (N_SIMD * cyc) if cyc else 0.0
        gflop = c.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) * 512 / 1e9
        short = name.split("(")[0].replace("void ", "")
        lines.append(f"| `{short}` | {len(dur[name])} | {ns:.0f} | {ghz:.2f} | {busy:.3f} | {gflop:.1f} | "
                     + " | ".join(f"{c.get(cn, float('nan')):.4g}" for cn in COUNTER_SET) + " |")
    return "\n".join(lines)


def summarize_pmc(db_path: str, substrs=("fa::",)) -> str:
    """Per-kernel means over dispatches of every counter a rocprofv3 --pmc
    pass collected (derived counters such as LdsUtil included), one column per
    counter in the order first seen."""
    import collections
    import sqlite3
    cur = sqlite3.connect(db_path).cursor()
    vals = collections.defaultdict(lambda: collections.defaultdict(lambda: collections.defaultdict(float)))
    names = []
    for name, did, cn, v in cur.execute(
            "select kernel_name, dispatch_id, counter_name, value from counters_collection"):
        vals[name][cn][did] += v
        if cn not in names:
            names.append(cn)
    lines = ["| kernel | dispatches | " + " | ".join(names) + " |", "|" + "---|" * (2 + len(names))]
    for name in sorted(vals):
        if not any(s in name for s in substrs):
            continue
        c = {cn: (sum(d.values()) / len(d), len(d)) for cn, d in vals[name].items()}
        nd = max(n for _, n in c.values())
        short = name.split("(")[0].replace("void ", "")
        lines.append(f"| `{short}` | {nd} | "
                     + " | ".join(f"{c[cn][0]:.4g}" if cn in c else "nan" for cn in names) + " |")
    return "\n".join(lines)


def summarize_traffic(fetch_db: str, write_db: str, workload: str, copy_bytes: int, update: bool) -> str:
    """HBM bytes per launch from FETCH_SIZE / WRITE_SIZE (KiB per dispatch),
    each scaled by what the same counter reads for a copy of copy_bytes."""
    fetch = _pmc_means(fetch_db, "FETCH_SIZE")
    write = _pmc_means(write_db, "WRITE_SIZE")
    cf = fetch.get(next((n for n in fetch if COPY_KERNEL in n), ""), None)
    cw = write.get(next((n for n in write if COPY_KERNEL in n), ""), None)
    if not cf or not cw:
        raise SystemExit("copy calibration kernel not found in the counter databases")
    f_scale = copy_bytes / (cf * 1024.0)      # true bytes per counted byte
    w_scale = copy_bytes / (cw * 1024.0)
    lines = [f"copy of {copy_bytes} B: FETCH_SIZE {cf:.0f} KiB (scale {f_scale:.4f}), "
             f"WRITE_SIZE {cw:.0f} KiB (scale {w_scale:.4f})", "",
             "| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM bytes per launch (scaled) |", "|---|---|---|---|"]
    rec = json.load(open(PROFILE_TRAFFIC)) if os.path.exists(PROFILE_TRAFFIC) else {}
    entry = rec.setdefault(workload, {})
    for sub, key in KEYS_BY_SUBSTR:
        fn = next((n for n in fetch if sub in n), None)
        wn = next((n for n in write if sub in n), None)
        if fn is None or wn is None:
            continue
        b = fetch[fn] * 1024.0 * f_scale + write[wn] * 1024.0 * w_scale
        lines.append(f"| `{fn}` | {fetch[fn]:.0f} | {write[wn]:.0f} | {b:.4g} |")
        entry[key] = {"hbm_bytes_per_launch": round(b), "fetch_kib": round(fetch[fn]), "write_kib": round(write[wn]),
                      "fetch_scale": round(f_scale, 5), "write_scale": round(w_scale, 5),
                      "source_digest": source_digest(*KERNEL_SOURCES[key])}
    if update:
        os.makedirs(os.path.dirname(PROFILE_TRAFFIC), exist_ok=True)
        json.dump(rec, open(PROFILE_TRAFFIC, "w"), indent=1, sort_keys=True)
    return "\n".join(lines)


STALL_SET_A = ("SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES", "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_WAIT_INST_LDS",
               "SQ_ACTIVE_INST_ANY", "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS")
STALL_SET_B = ("SQ_ACTIVE_INST_MISC", "SQ_ACTIVE_INST_VMEM", "SQ_ACTIVE_INST_SCA", "SQ_INSTS_VALU", "SQ_INSTS_LDS",
               "SQ_INSTS_SALU", "SQ_ACTIVE_INST_VALU2", "SQ_INSTS_MFMA")


def summarize_stalls(db_paths, substrs=("fa::",)) -> str:
    """Where each kernel's waves spend their cycles, from the STALL_SET_A
    pass (and optionally STALL_SET_B): the shares of SQ_WAVE_CYCLES spent
    issuing (SQ_ACTIVE_INST_ANY), waiting on a dependency such as s_waitcnt
    or a barrier (SQ_WAIT_ANY) and ready but not issued (SQ_WAIT_INST_ANY);
    the three partition a wave's life. Also the vector and LDS issue shares
    and, with the second pass, instructions per MFMA."""
    import collections
    import sqlite3
    vals = collections.defaultdict(lambda: collections.defaultdict(lambda: collections.defaultdict(float)))
    for db in db_paths:
        cur = sqlite3.connect(db).cursor()
        for name, did, cn, v in cur.execute(
                "select kernel_name, dispatch_id, counter_name, value from counters_collection"):
            vals[name][cn][did] += v
    lines = ["| kernel | issuing | waiting on a dependency | waiting for issue | VALU active | LDS active | "
             "VALU instr. per MFMA | LDS instr. per MFMA |", "|---|---|---|---|---|---|---|---|"]
    for name in sorted(vals):
        if not any(x in name for x in substrs):
            continue
        c = {cn: sum(d.values()) / len(d) for cn, d in vals[name].items()}
        wc = c.get("SQ_WAVE_CYCLES", 0.0)
        if not wc:
            continue
        share = lambda k: f"{100.0 * c[k] / wc:.1f} %" if k in c else "—"
        mf = c.get("SQ_INSTS_MFMA", 0.0)
        per = lambda k: f"{c[k] / mf:.2f}" if mf and k in c else "—"
        short = name.split("(")[0].replace("void ", "")
        lines.append(f"| `{short}` | {share('SQ_ACTIVE_INST_ANY')} | {share('SQ_WAIT_ANY')} | "
                     f"{share('SQ_WAIT_INST_ANY')} | {share('SQ_ACTIVE_INST_VALU')} | {share('SQ_ACTIVE_INST_LDS')} | "
                     f"{per('SQ_INSTS_VALU')} | {per('SQ_INSTS_LDS')} |")
    return "\n".join(lines)


def _pmc_sums(db_path: str, counter: str) -> dict:
    """Counter totals per kernel name over all its dispatches."""
    import collections
    import sqlite3
    cur = sqlite3.connect(db_path).cursor()
    tot = collections.defaultdict(float)
    for name, val in cur.execute("select kernel_name, value from counters_collection where counter_name = ?",
                                 (counter,)):
        tot[name] += val
    return tot


def summarize_step_traffic(fetch_db: str, write_db: str, copy_bytes: int, steps: int) -> str:
    """HBM bytes per step of a run: FETCH_SIZE + WRITE_SIZE summed over every
    kernel except the device copies and fills, scaled by the calibration copy,
    divided by the number of steps the run made."""
    fetch, write = _pmc_sums(fetch_db, "FETCH_SIZE"), _pmc_sums(write_db, "WRITE_SIZE")
    cf = _pmc_means(fetch_db, "FETCH_SIZE").get(next((n for n in fetch if COPY_KERNEL in n), ""), None)
    cw = _pmc_means(write_db, "WRITE_SIZE").get(next((n for n in write if COPY_KERNEL in n), ""), None)
    if not cf or not cw:
        raise SystemExit("copy calibration kernel not found in the counter databases")
    f_scale, w_scale = copy_bytes / (cf * 1024.0), copy_bytes / (cw * 1024.0)
    # the calibration copy and its source fill; the comparator's mask, built once before the steps
    skip = (COPY_KERNEL, "__amd_rocclr_fill", "FillFunctor<unsigned char>", "FillFunctor<bool>", "triu_tril")
    lines = [f"copy of {copy_bytes} B: FETCH_SIZE scale {f_scale:.4f}, WRITE_SIZE scale {w_scale:.4f}; {steps} steps",
             "", "| kernel | FETCH GB per step | WRITE GB per step |", "|---|---|---|"]
    tf = tw = 0.0
    for n in sorted(set(fetch) | set(write)):
        if any(x in n for x in skip):
            continue
        fb = fetch.get(n, 0.0) * 1024.0 * f_scale / steps
        wb = write.get(n, 0.0) * 1024.0 * w_scale / steps
        tf, tw = tf + fb, tw + wb
        lines.append(f"| `{n[:120]}` | {fb / 1e9:.3f} | {wb / 1e9:.3f} |")
    lines += ["", f"Total per step: {tf / 1e9:.2f} GB read + {tw / 1e9:.2f} GB written = {(tf + tw) / 1e9:.2f} GB"]
    return "\n".join(lines)


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="long_prefill",
                    choices=sorted(synth.WORKLOADS) + sorted(synth.PACKED_WORKLOADS) + sorted(synth.FP8_WORKLOADS))
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle time for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-naive", action="store_true")
    ap.add_argument("--no-also", action="store_true",
                    help="skip the secondary forward + backward record of forward-only workloads")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="after the run, copy BYTES once more between two device buffers (counter calibration)")
    ap.add_argument("--summarize-trace", metavar="DB", help="print a kernel table from a rocprofv3 trace database")
    ap.add_argument("--summarize-traffic", nargs=2, metavar=("FETCH_DB", "WRITE_DB"),
                    help="HBM bytes per launch from FETCH_SIZE / WRITE_SIZE counter databases")
    ap.add_argument("--copy-bytes", type=int, default=1 << 30)
    ap.add_argument("--update-traffic", action="store_true", help="write the result into profiles/traffic.json")
    ap.add_argument("--sweep", action="store_true",
                    help="fwd and fwd+bwd TFLOP/s over N = 1K..32K (B*N = 32K tokens, H = 16), d = 64/128, "
                         "no mask and causal; one JSON line per point, then a markdown table")
    ap.add_argument("--tile-sweep", action="store_true",
                    help="forward runtime against the query rows per workgroup (32..256) on the GPT-2-medium "
                         "and causal training shapes, next to the tile-model HBM bytes")
    ap.add_argument("--summarize-kernel-traffic", nargs=3, metavar=("FETCH_DB", "WRITE_DB", "SUBSTR"),
                    help="scaled HBM bytes per dispatch of every kernel whose name holds SUBSTR")
    ap.add_argument("--naive-only", action="store_true",
                    help="run only the materialise-S comparator, warmup + steps times (for its counter passes)")
    ap.add_argument("--summarize-step-traffic", nargs=3, metavar=("FETCH_DB", "WRITE_DB", "STEPS"),
                    help="scaled HBM bytes per step summed over every kernel of a run (copies excluded)")
    ap.add_argument("--summarize-stalls", nargs="+", metavar="DB",
                    help="per-kernel shares of wave cycles (issuing / waiting on a dependency / waiting for issue) "
                         "from the stall counter passes")
    ap.add_argument("--atomic-rate", action="store_true",
                    help="fp32 atomic-add throughput (torch index_add_), each address updated 1, 8 or 32 times: "
                         "the rate an atomic dQ accumulation would run at")
    ap.add_argument("--summarize-counters", metavar="DB",
                    help="per-kernel table (clock, MFMA busy, executed MFMA FLOPs, ...) from a counter pass")
    ap.add_argument("--summarize-pmc", metavar="DB",
                    help="per-kernel means of every counter in a rocprofv3 --pmc pass (e.g. LdsUtil, LdsLatency)")
    args = ap.parse_args()

    if args.summarize_step_traffic:
        f_db, w_db, steps = args.summarize_step_traffic
        print(summarize_step_traffic(f_db, w_db, args.copy_bytes, int(steps)))
        return 0
    if args.summarize_pmc:
        print(summarize_pmc(args.summarize_pmc))
        return 0
    if args.summarize_counters:
        print(summarize_counters(args.summarize_counters))
        return 0
    if args.summarize_stalls:
        print(summarize_stalls(args.summarize_stalls))
        return 0
    if args.summarize_kernel_traffic:
        f_db, w_db, sub = args.summarize_kernel_traffic
        print(summarize_kernel_traffic(f_db, w_db, args.copy_bytes, sub))
        return 0
    if args.summarize_trace:
        print(summarize_trace(args.summarize_trace))
        return 0
    if args.summarize_traffic:
        print(summarize_traffic(*args.summarize_traffic, args.workload, args.copy_bytes, args.update_traffic))
        return 0

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(heads are independent; sharding them needs no communication). Run with --gpus 1.",
              file=sys.stderr)
        return 2

    import torch
    import io_aware_exact_10_amd as fa

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        return 1
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.sweep:
        return run_sweep(args, dev)
    if args.atomic_rate:
        return run_atomic_rate(dev)
    if args.tile_sweep:
        return run_tile_sweep(args, dev)
    if args.workload in synth.PACKED_WORKLOADS:
        return run_packed(args, synth.PACKED_WORKLOADS[args.workload], dev)
    if args.workload in synth.FP8_WORKLOADS:
        return run_fp8(args, synth.FP8_WORKLOADS[args.workload], dev)
    w = synth.WORKLOADS[args.workload]
    backward = w.backward
    print(f"# workload {w.name}: B{w.B} H{w.H} N{w.N} d{w.d} dtype{w.dtype} mask{w.mask_kind} "
          f"{'fwd+bwd' if backward else 'fwd'}", file=sys.stderr, flush=True)
    inp = synth.make_inputs(w)

    def dev_t(vals, bits):
        if w.dtype == synth.DTYPE_BF16:
            return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(vals).to(dev)

    q, k, v = dev_t(inp.q, inp.q_bits), dev_t(inp.k, inp.k_bits), dev_t(inp.v, inp.v_bits)
    do = dev_t(inp.do, inp.do_bits) if backward else None
    mask_t = torch.from_numpy(inp.mask).to(dev) if inp.mask is not None else None
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
    if backward:
        dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
        ws = torch.empty(fa.fa_bwd_workspace_bytes(w.B, w.H, w.N, w.d), dtype=torch.uint8, device=dev)

    def step():
        fa.forward(q, k, v, w.scale, w.mask_kind, mask_t, out=o, lse=lse)
        if backward:
            fa.backward(q, k, v, o, lse, do, w.scale, w.mask_kind, mask_t, workspace=ws, dq=dq, dk=dk, dv=dv)

    if args.naive_only:
        # Only the comparator, warmup + steps times (for a counter pass over its kernels).
        bm = naive_mask(w, mask_t, dev)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.warmup + args.steps):
            naive_full(q, k, v, do, w.scale, w.mask_kind, bm, backward)
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / max(1, args.warmup + args.steps)
        copy_calibration(args.copy_calibration, dev)
        print(json.dumps({"naive_only": w.name, "steps": args.warmup + args.steps, "wall_ms_per_step": round(ms, 3)}))
        return 0

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"# warmup done ({args.warmup} steps)", file=sys.stderr, flush=True)

    # The timed step enqueues fa_fwd and the three steps of fa_bwd one by one,
    # with a HIP event between launches on the launch stream.
    stream = torch.cuda.current_stream(dev)
    names = ["fwd"] + (["rowterm", "dkdv", "dq"] if backward else [])
    per, wall = time_dense(fa, stream, q, k, v, do, o, lse, w.scale, w.mask_kind, mask_t,
                           (ws, dq, dk, dv) if backward else None, args.steps)
    fwd_ms = per["fwd"]
    bwd_ms = sum(per[n] for n in names[1:]) if backward else np.zeros_like(fwd_ms)
    step_ms = fwd_ms + bwd_ms
    print(f"# timed {args.steps} steps: {step_ms.mean():.3f} ms/step (wall {wall * 1e3 / args.steps:.3f}) "
          + " ".join(f"{n} {per[n].mean():.3f}" for n in names), file=sys.stderr, flush=True)

    vis = visible_pairs(w, inp.mask)
    heads = w.B * w.H
    fwd_flop = 4.0 * w.d * vis * heads
    bwd_flop = 10.0 * w.d * vis * heads if backward else 0.0
    ms_per_step = float(step_ms.mean())
    value = (fwd_flop + bwd_flop) / (ms_per_step * 1e-3) / 1e12
    fwd_tflops = fwd_flop / (fwd_ms.mean() * 1e-3) / 1e12
    bwd_tflops = bwd_flop / (bwd_ms.mean() * 1e-3) / 1e12 if backward else None

    peak = PEAK_BF16_TFLOPS if w.dtype == synth.DTYPE_BF16 else PEAK_F32_VALU_TFLOPS
    kflop = {"fwd": fwd_flop, "rowterm": 0.0, "dkdv": 8.0 * w.d * vis * heads, "dq": 2.0 * w.d * vis * heads}
    kname = dict(KERNEL_NAMES) if w.dtype == synth.DTYPE_BF16 else {n: KERNEL_NAMES[n].replace("_bf16_", "_f32_")
                                                                    for n in names}
    if w.dtype == synth.DTYPE_BF16 and w.d == 128:
        kname["dkdv"] = "bwd_dkdv8_bf16_kernel"     # the eight-wave dK/dV kernel at d = 128
    kernels = {}
    for n in names:
        t = float(per[n].mean())
        kernels[n] = {"kernel": kname[n], "mean_ms": round(t, 4), "median_ms": round(float(np.median(per[n])), 4),
                      "min_ms": round(float(per[n].min()), 4), "algorithmic_gflop": round(kflop[n] / 1e9, 2),
                      "tflops": round(kflop[n] / (t * 1e-3) / 1e12, 2),
                      "hbm_gbs": hbm_rate(measured_traffic(w.name, n), t)}
    dom = max((n for n in names if n != "rowterm"), key=lambda n: per[n].mean())
    dom_t = float(per[dom].mean())
    achieved = kflop[dom] / (dom_t * 1e-3) / 1e12
    traffic = measured_traffic(w.name, dom)
    roofline = {"kernel": kname[dom],
                "bound": "mfma" if w.dtype == synth.DTYPE_BF16 else "alu",
                "achieved": round(achieved, 2), "peak": round(peak, 1), "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4), "traffic": traffic, "traffic_gbs": hbm_rate(traffic, dom_t),
                "flop_per_launch": kflop[dom], "mean_launch_ms": round(dom_t, 4),
                "median_launch_ms": round(float(np.median(per[dom])), 4),
                "frac_at_median": round(kflop[dom] / (float(np.median(per[dom])) * 1e-3) / 1e12 / peak, 4)}

    naive = None
    if not args.no_naive:
        try:
            bm = naive_mask(w, mask_t, dev)
            for _ in range(2):
                naive_full(q, k, v, do, w.scale, w.mask_kind, bm, backward)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            reps = 3
            e0.record(stream)
            for _ in range(reps):
                naive_full(q, k, v, do, w.scale, w.mask_kind, bm, backward)
            e1.record(stream)
            torch.cuda.synchronize()
            nms = e0.elapsed_time(e1) / reps
            naive = {"ms_per_step": round(nms, 3), "tflops": round((fwd_flop + bwd_flop) / (nms * 1e-3) / 1e12, 2),
                     "what": "torch matmul, mask, softmax (fp32), matmul" + ("; autograd backward" if backward else "")
                             + ("; one head at a time" if w.N > NAIVE_WHOLE_N else "")}
        except Exception as ex:  # noqa: BLE001
            naive = {"error": repr(ex)[:200]}
        torch.cuda.empty_cache()

    copy_calibration(args.copy_calibration, dev)

    cpu = None
    if not args.no_cpu_baseline:
        print("# timing the CPU oracle sample", file=sys.stderr, flush=True)
        flop_head = (fwd_flop + bwd_flop) / heads
        cpu = cpu_baseline(inp, args.cpu_budget, backward, flop_head)

    also = None
    if not backward and not args.no_also and w.dtype == synth.DTYPE_BF16:
        del q, k, v, o, lse
        torch.cuda.empty_cache()
        also = time_fwd_bwd_device_inputs(fa, stream, synth.WORKLOADS["causal_train"], args.steps, args.warmup, dev)

    what = "fwd+bwd" if backward else "fwd"
    mask_name = {0: "none", 1: "causal", 2: "block-sparse"}[w.mask_kind]
    rec = {
        "metric": "attention fwd / fwd+bwd TFLOP/s and % of bf16 MFMA peak, N=1k-32k, d=64/128",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        # The pages publish no number for this metric on this hardware; their
        # A100 runtime of the GPT-2-medium shape is context only (below).
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == synth.DTYPE_BF16 else "f32",
        "data": "synthetic: Q, K, V, dO ~ N(0,1) seeded, bf16 round-to-nearest-even",
        "config": {"workload": f"{w.name}: B={w.B} H={w.H} N={w.N} d={w.d} mask={mask_name} {what}",
                   "B": w.B, "H": w.H, "N": w.N, "d": w.d, "mask": mask_name, "pass": what,
                   "seed": w.seed, "scale": w.scale},
        "frac_of_peak": round(value / peak, 4),
        "step_ms": {"mean": round(ms_per_step, 4), "median": round(float(np.median(step_ms)), 4),
                    "min": round(float(step_ms.min()), 4)},
        "fwd": {"ms": round(float(fwd_ms.mean()), 4), "median_ms": round(float(np.median(fwd_ms)), 4),
                "min_ms": round(float(fwd_ms.min()), 4), "tflops": round(fwd_tflops, 2),
                "frac": round(fwd_tflops / peak, 4), "gflop": round(fwd_flop / 1e9, 2)},
        "bwd": ({"ms": round(float(bwd_ms.mean()), 4), "median_ms": round(float(np.median(bwd_ms)), 4),
                 "min_ms": round(float(bwd_ms.min()), 4), "tflops": round(bwd_tflops, 2),
                 "frac": round(bwd_tflops / peak, 4), "gflop": round(bwd_flop / 1e9, 2)} if backward else None),
        "kernels": kernels,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "naive": naive,
        "speedup_vs_naive": (round(naive["ms_per_step"] / ms_per_step, 2)
                             if naive and "ms_per_step" in naive else None),
        "context_a100_fig2_ms": A100_FIG2_MS if w.name == "gpt2_medium" else None,
        "also": also,
        "wall_ms_per_step": round(wall * 1e3 / args.steps, 4),
    }
    print(json.dumps(rec), flush=True)
    return 0


def time_dense(fa, stream, q, k, v, do, o, lse, scale, mask_kind, mask_t, bwd_bufs, steps):
    """Times ``steps`` steps: fa_fwd, then (with ``bwd_bufs`` = (workspace,
    dq, dk, dv)) the three steps of fa_bwd enqueued one by one, with a HIP
    event on the launch stream between launches. Returns the per-kernel
    durations in ms (arrays over the steps) and the wall time in s."""
    import torch
    names = ["fwd"] + (["rowterm", "dkdv", "dq"] if bwd_bufs is not None else [])
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        ev[i][0].record(stream)
        fa.forward(q, k, v, scale, mask_kind, mask_t, out=o, lse=lse)
        ev[i][1].record(stream)
        if bwd_bufs is not None:
            ws, dq, dk, dv = bwd_bufs
            for j, st in enumerate(("rowterm", "dkdv", "dq")):
                fa.backward(q, k, v, o, lse, do, scale, mask_kind, mask_t, workspace=ws, dq=dq, dk=dk, dv=dv,
                            steps=st)
                ev[i][2 + j].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = {n: np.array([ev[i][j].elapsed_time(ev[i][j + 1]) for i in range(steps)]) for j, n in enumerate(names)}
    return per, wall


def time_fwd_bwd_device_inputs(fa, stream, w: synth.Workload, steps: int, warmup: int, dev) -> dict:
    """Forward + backward of workload ``w`` (no block mask) on N(0, 1) bf16
    inputs drawn on the device from a seeded generator (timing only: the
    parity tests cover these shapes on the host-drawn inputs)."""
    import torch
    gen = torch.Generator(device=dev)
    gen.manual_seed(w.seed)
    shape = (w.B, w.H, w.N, w.d)
    q, k, v, do = (torch.randn(shape, generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
                   for _ in range(4))
    o = torch.empty_like(q)
    lse = torch.empty(shape[:3], dtype=torch.float32, device=dev)
    bufs = (torch.empty(fa.fa_bwd_workspace_bytes(*shape), dtype=torch.uint8, device=dev),
            torch.empty_like(q), torch.empty_like(q), torch.empty_like(q))
    for _ in range(warmup):
        time_dense(fa, stream, q, k, v, do, o, lse, w.scale, w.mask_kind, None, bufs, 1)
    per, _ = time_dense(fa, stream, q, k, v, do, o, lse, w.scale, w.mask_kind, None, bufs, steps)
    vis = visible_pairs(w, None)
    heads = w.B * w.H
    kflop = {"fwd": 4.0 * w.d * vis * heads, "rowterm": 0.0, "dkdv": 8.0 * w.d * vis * heads,
             "dq": 2.0 * w.d * vis * heads}
    step = sum(per.values())
    tf = 14.0 * w.d * vis * heads / (step.mean() * 1e-3) / 1e12
    mask_name = {0: "none", 1: "causal"}[w.mask_kind]
    out = {"workload": f"{w.name}: B={w.B} H={w.H} N={w.N} d={w.d} mask={mask_name} fwd+bwd",
           "ms_per_step": round(float(step.mean()), 4), "median_ms": round(float(np.median(step)), 4),
           "tflops": round(tf, 2), "frac": round(tf / PEAK_BF16_TFLOPS, 4),
           "kernels": {n: {"mean_ms": round(float(per[n].mean()), 4),
                           "tflops": round(kflop[n] / (per[n].mean() * 1e-3) / 1e12, 2)} for n in per}}
    print(f"# also {out['workload']}: {out['ms_per_step']} ms/step, {out['tflops']} TFLOP/s", file=sys.stderr,
          flush=True)
    del q, k, v, do, o, lse, bufs
    torch.cuda.empty_cache()
    return out


def run_packed(args, w: synth.PackedWorkload, dev) -> int:
    """Packed variable-length batch with shared K/V heads: fa_fwd_varlen then
    fa_bwd_varlen per step (the backward's three kernels in one call)."""
    import torch
    import io_aware_exact_10_amd as fa

    lens = w.lengths()
    qlens = w.query_lengths()
    print(f"# workload {w.name}: B{w.B} key lengths {lens} query lengths {qlens[:4]}... H{w.H} Hkv{w.Hkv} d{w.d} "
          f"mask{w.mask_kind}", file=sys.stderr, flush=True)
    if w.queries:
        return run_decode(args, w, lens, qlens, dev)
    p = synth.packed_inputs(lens, lens, w.H, w.Hkv, w.d, w.seed)

    def dev_t(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    q, k, v, do = dev_t(p.q_bits), dev_t(p.k_bits), dev_t(p.v_bits), dev_t(p.do_bits)
    cu = torch.from_numpy(p.cu_q).to(dev)
    mx = max(lens)
    Tq = q.shape[0]
    o = torch.empty_like(q)
    lse = torch.empty((w.H, Tq), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(fa.fa_bwd_varlen_workspace_bytes(Tq, w.H, w.d), dtype=torch.uint8, device=dev)

    def fwd():
        fa.forward_varlen(q, k, v, cu, cu, mx, mx, w.scale, w.mask_kind, out=o, lse=lse)

    def bwd():
        fa.backward_varlen(q, k, v, o, lse, do, cu, cu, mx, mx, w.scale, w.mask_kind, workspace=ws,
                           dq=dq, dk=dk, dv=dv)

    for _ in range(args.warmup):
        fwd()
        if w.backward:
            bwd()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record(stream)
        fwd()
        ev[i][1].record(stream)
        if w.backward:
            bwd()
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    fwd_ms = np.array([e[0].elapsed_time(e[1]) for e in ev])
    bwd_ms = np.array([e[1].elapsed_time(e[2]) for e in ev])
    step_ms = fwd_ms + bwd_ms
    print(f"# timed {args.steps} steps: {step_ms.mean():.3f} ms/step fwd {fwd_ms.mean():.3f} bwd {bwd_ms.mean():.3f}",
          file=sys.stderr, flush=True)
    copy_calibration(args.copy_calibration, dev)
    if w.mask_kind == synth.MASK_CAUSAL:
        vis = sum(n * (n + 1) // 2 for n in lens)
    else:
        vis = sum(n * n for n in lens)
    fwd_flop = 4.0 * w.d * vis * w.H
    bwd_flop = 10.0 * w.d * vis * w.H if w.backward else 0.0
    ms = float(step_ms.mean())
    value = (fwd_flop + bwd_flop) / (ms * 1e-3) / 1e12
    fwd_tf = fwd_flop / (fwd_ms.mean() * 1e-3) / 1e12
    bwd_tf = bwd_flop / (bwd_ms.mean() * 1e-3) / 1e12 if w.backward else None

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        print("# timing the CPU oracle sample", file=sys.stderr, flush=True)
        t1 = time.perf_counter()
        G = w.H // w.Hkv
        done, flops = 0, 0.0
        for b, n in enumerate(lens):
            a, e = int(p.cu_q[b]), int(p.cu_q[b + 1])
            for h in range(w.H):
                oracle.forward_head(p.q[a:e, h], p.k[a:e, h // G], p.v[a:e, h // G], w.scale, w.mask_kind)
                if w.backward:
                    oracle.backward_head(p.q[a:e, h], p.k[a:e, h // G], p.v[a:e, h // G], p.do[a:e, h], w.scale,
                                         w.mask_kind)
                done += 1
                pairs = n * (n + 1) // 2 if w.mask_kind == synth.MASK_CAUSAL else n * n
                flops += (14.0 if w.backward else 4.0) * w.d * pairs
                if time.perf_counter() - t1 > args.cpu_budget:
                    break
            if time.perf_counter() - t1 > args.cpu_budget:
                break
        el = time.perf_counter() - t1
        cpu = {"value": flops / el / 1e12, "unit": "TFLOP/s", "cores": len(os.sched_getaffinity(0)),
               "kind": "oracle", "sample": f"{done} (sequence, head) pairs of {w.B * w.H}", "seconds": round(el, 2)}

    mask_name = {0: "none", 1: "causal"}[w.mask_kind]
    what = "fwd+bwd" if w.backward else "fwd"
    rec = {
        "metric": "attention fwd / fwd+bwd TFLOP/s and % of bf16 MFMA peak, N=1k-32k, d=64/128",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic: Q, K, V, dO ~ N(0,1) seeded, bf16 round-to-nearest-even; "
                                 "sequence lengths uniform in [max/8, max]",
        "config": {"workload": f"{w.name}: packed B={w.B} max_len={w.max_len} tokens={Tq} H={w.H} Hkv={w.Hkv} "
                               f"d={w.d} mask={mask_name} {what}",
                   "lengths": lens, "H": w.H, "Hkv": w.Hkv, "d": w.d, "mask": mask_name, "pass": what,
                   "seed": w.seed},
        "frac_of_peak": round(value / PEAK_BF16_TFLOPS, 4),
        "fwd": {"ms": round(float(fwd_ms.mean()), 4), "tflops": round(fwd_tf, 2),
                "frac": round(fwd_tf / PEAK_BF16_TFLOPS, 4), "gflop": round(fwd_flop / 1e9, 2)},
        "bwd": ({"ms": round(float(bwd_ms.mean()), 4), "tflops": round(bwd_tf, 2),
                 "frac": round(bwd_tf / PEAK_BF16_TFLOPS, 4), "gflop": round(bwd_flop / 1e9, 2)}
                if w.backward else None),
        "roofline": {"kernel": KERNEL_NAMES["fwd"], "bound": "mfma", "achieved": round(fwd_tf, 2),
                     "peak": round(PEAK_BF16_TFLOPS, 1), "unit": "TFLOP/s", "frac": round(fwd_tf / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic(w.name, "fwd"),
                     "traffic_gbs": hbm_rate(measured_traffic(w.name, "fwd"), float(fwd_ms.mean())),
                     "flop_per_launch": fwd_flop, "mean_launch_ms": round(float(fwd_ms.mean()), 4)},
        "cpu_baseline": cpu,
        "wall_ms_per_step": round(wall * 1e3 / args.steps, 4),
    }
    print(json.dumps(rec), flush=True)
    return 0


def run_atomic_rate(dev) -> int:
    """Device-wide throughput of fp32 atomic adds (index_add_ with repeated
    indices: every address receives `adds` updates, as a dQ accumulator
    would from the key tiles of one query tile). Each update also reads its
    8-byte index and 4-byte source value. HIP-event medians."""
    import torch
    n = 1 << 23                                          # 32 MiB of fp32 accumulators
    acc = torch.zeros(n, dtype=torch.float32, device=dev)
    out = []
    for adds in (1, 8, 32):
        idx = torch.arange(n, device=dev, dtype=torch.int64).repeat(adds)
        src = torch.ones(n * adds, dtype=torch.float32, device=dev)
        for _ in range(3):
            acc.index_add_(0, idx, src)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(5)]
        for e0, e1 in ev:
            e0.record()
            acc.index_add_(0, idx, src)
            e1.record()
        torch.cuda.synchronize()
        ms = float(np.median([e0.elapsed_time(e1) for e0, e1 in ev]))
        rec = {"updates_per_address": adds, "ms": round(ms, 4),
               "atomic_updates_tb_s": round(n * adds * 4 / (ms * 1e-3) / 1e12, 3)}
        out.append(rec)
        print(json.dumps(rec), flush=True)
        del idx, src
    print("| updates per address | ms | fp32 atomic updates (TB/s) |")
    print("|---|---|---|")
    for r in out:
        print(f"| {r['updates_per_address']} | {r['ms']} | {r['atomic_updates_tb_s']} |")
    return 0


def run_sweep(args, dev) -> int:
    """Sequence-length sweep at a fixed token count (B * N = 32768, H = 16):
    seeded N(0, 1) bf16 inputs drawn on the device; forward and forward +
    backward timed with HIP events (median over the timed steps)."""
    import torch
    import io_aware_exact_10_amd as fa

    gen = torch.Generator(device=dev)
    rows = []
    for d in (64, 128):
        for mask_kind in (synth.MASK_NONE, synth.MASK_CAUSAL):
            for N in (1024, 2048, 4096, 8192, 16384, 32768):
                B, H = 32768 // N, 16
                gen.manual_seed(1000 * d + 10 * mask_kind + N)
                q, k, v, do = (torch.randn((B, H, N, d), generator=gen, device=dev, dtype=torch.float32)
                               .to(torch.bfloat16) for _ in range(4))
                o = torch.empty_like(q)
                lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
                dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
                ws = torch.empty(fa.fa_bwd_workspace_bytes(B, H, N, d), dtype=torch.uint8, device=dev)
                scale = 1.0 / math.sqrt(d)

                def fwd():
                    fa.forward(q, k, v, scale, mask_kind, None, out=o, lse=lse)

                def bwd():
                    fa.backward(q, k, v, o, lse, do, scale, mask_kind, None, workspace=ws, dq=dq, dk=dk, dv=dv)

                for _ in range(args.warmup):
                    fwd()
                    bwd()
                torch.cuda.synchronize()
                ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
                for i in range(args.steps):
                    ev[i][0].record()
                    fwd()
                    ev[i][1].record()
                    bwd()
                    ev[i][2].record()
                torch.cuda.synchronize()
                f_ms = float(np.median([e[0].elapsed_time(e[1]) for e in ev]))
                b_ms = float(np.median([e[1].elapsed_time(e[2]) for e in ev]))
                vis = N * N if mask_kind == synth.MASK_NONE else N * (N + 1) // 2
                fl = 4.0 * d * vis * B * H
                rec = {"N": N, "B": B, "H": H, "d": d, "mask": "causal" if mask_kind else "none",
                       "fwd_ms": round(f_ms, 4), "fwd_tflops": round(fl / (f_ms * 1e-3) / 1e12, 1),
                       "fwd_frac": round(fl / (f_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                       "fwdbwd_ms": round(f_ms + b_ms, 4),
                       "fwdbwd_tflops": round(3.5 * fl / ((f_ms + b_ms) * 1e-3) / 1e12, 1)}
                rows.append(rec)
                print(json.dumps(rec), flush=True)
                del q, k, v, do, o, lse, dq, dk, dv, ws
                torch.cuda.empty_cache()
    print("| d | mask | N | B | fwd ms | fwd TFLOP/s | % of bf16 peak | fwd+bwd ms | fwd+bwd TFLOP/s |")
    print("|---|---|---|---|---|---|---|---|---|")
    for r in rows:
        print(f"| {r['d']} | {r['mask']} | {r['N']} | {r['B']} | {r['fwd_ms']} | {r['fwd_tflops']} | "
              f"{100 * r['fwd_frac']:.1f} | {r['fwdbwd_ms']} | {r['fwdbwd_tflops']} |")
    return 0


TILE_SWEEP_SHAPES = (
    # name, B, H, N, d, mask kind
    ("gpt2_medium", 64, 16, 1024, 64, synth.MASK_NONE),
    ("causal_train", 8, 16, 4096, 128, synth.MASK_CAUSAL),
)
TILE_SWEEP_ROWS = (32, 64, 128, 256)


def tile_model_bytes(N: int, d: int, rows: int, causal: bool, e: int = 2) -> int:
    """HBM bytes per head the forward's schedule implies with no cache reuse:
    Q read and O written once, the LSE written once, and every workgroup of
    `rows` queries reading the 64-key K and V tiles its rows see."""
    kv = 0
    for t in range((N + rows - 1) // rows):
        keys = min(N, (t + 1) * rows) if causal else N
        keys = min(N, (keys + 63) // 64 * 64)
        kv += 2 * keys * d * e
    return 2 * N * d * e + kv + 4 * N


def run_tile_sweep(args, dev) -> int:
    """Forward runtime against the query rows per workgroup (fa_fwd_tiled,
    32..256 rows, 64-key tiles) on the GPT-2-medium shape and the causal
    training shape: HIP-event medians over the timed steps, next to the
    schedule's own HBM byte count (tile model, no cache reuse)."""
    import torch
    import io_aware_exact_10_amd as fa

    gen = torch.Generator(device=dev)
    rows_out = []
    for name, B, H, N, d, mask_kind in TILE_SWEEP_SHAPES:
        gen.manual_seed(5000 + N + d)
        q, k, v = (torch.randn((B, H, N, d), generator=gen, device=dev, dtype=torch.float32)
                   .to(torch.bfloat16) for _ in range(3))
        o = torch.empty_like(q)
        lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
        scale = 1.0 / math.sqrt(d)
        vis = N * N if mask_kind == synth.MASK_NONE else N * (N + 1) // 2
        fl = 4.0 * d * vis * B * H
        for br in TILE_SWEEP_ROWS:
            def fwd():
                fa.forward(q, k, v, scale, mask_kind, None, out=o, lse=lse, block_rows=br)

            for _ in range(args.warmup):
                fwd()
            torch.cuda.synchronize()
            ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
            for i in range(args.steps):
                ev[i][0].record()
                fwd()
                ev[i][1].record()
            torch.cuda.synchronize()
            ms = float(np.median([e[0].elapsed_time(e[1]) for e in ev]))
            model = tile_model_bytes(N, d, br, mask_kind == synth.MASK_CAUSAL) * B * H
            rec = {"shape": name, "B": B, "H": H, "N": N, "d": d, "mask": "causal" if mask_kind else "none",
                   "block_rows": br, "fwd_ms": round(ms, 4), "tflops": round(fl / (ms * 1e-3) / 1e12, 1),
                   "tile_model_gb": round(model / 1e9, 3)}
            rows_out.append(rec)
            print(json.dumps(rec), flush=True)
        del q, k, v, o, lse
        torch.cuda.empty_cache()
    copy_calibration(args.copy_calibration, dev)
    print("| shape | rows per workgroup | fwd ms | TFLOP/s | tile-model HBM GB |")
    print("|---|---|---|---|---|")
    for r in rows_out:
        print(f"| {r['shape']} (B={r['B']} H={r['H']} N={r['N']} d={r['d']} {r['mask']}) | {r['block_rows']} | "
              f"{r['fwd_ms']} | {r['tflops']} | {r['tile_model_gb']} |")
    return 0


def summarize_kernel_traffic(fetch_db: str, write_db: str, copy_bytes: int, substr: str) -> str:
    """Scaled HBM bytes per dispatch for every kernel whose name holds substr."""
    fetch = _pmc_means(fetch_db, "FETCH_SIZE")
    write = _pmc_means(write_db, "WRITE_SIZE")
    cf = fetch.get(next((n for n in fetch if COPY_KERNEL in n), ""), None)
    cw = write.get(next((n for n in write if COPY_KERNEL in n), ""), None)
    if not cf or not cw:
        raise SystemExit("copy calibration kernel not found in the counter databases")
    f_scale, w_scale = copy_bytes / (cf * 1024.0), copy_bytes / (cw * 1024.0)
    lines = [f"copy of {copy_bytes} B: FETCH_SIZE scale {f_scale:.4f}, WRITE_SIZE scale {w_scale:.4f}", "",
             "| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM GB per launch (scaled) |", "|---|---|---|---|"]
    for n in sorted(fetch):
        if substr in n and n in write:
            b = fetch[n] * 1024.0 * f_scale + write[n] * 1024.0 * w_scale
            lines.append(f"| `{n}` | {fetch[n]:.0f} | {write[n]:.0f} | {b / 1e9:.3f} |")
    return "\n".join(lines)


def run_fp8(args, w: synth.Workload, dev) -> int:
    """FP8 (E4M3) forward: fa_fwd_fp8 per step on codes drawn by
    synth.fp8_inputs (V transposed); FLOPs 4*d*vis per head."""
    import torch
    import io_aware_exact_10_amd as fa

    print(f"# workload {w.name}: B{w.B} H{w.H} N{w.N} d{w.d} fp8 mask{w.mask_kind} fwd", file=sys.stderr, flush=True)
    f = synth.fp8_inputs(w.B, w.H, w.N, w.d, w.seed)
    q8, k8, vt8 = (torch.from_numpy(x).to(dev) for x in (f.q8, f.k8, f.vt8))
    o = torch.empty((w.B, w.H, w.N, w.d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)

    def fwd():
        fa.forward_fp8(q8, k8, vt8, f.q_descale, f.k_descale, f.v_descale, w.scale, w.mask_kind, out=o, lse=lse)

    for _ in range(args.warmup):
        fwd()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record(stream)
        fwd()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    copy_calibration(args.copy_calibration, dev)
    vis = visible_pairs(w, None)
    flop = 4.0 * w.d * vis * w.B * w.H
    tf = flop / (ms * 1e-3) / 1e12
    print(f"# timed {args.steps} steps: {ms:.4f} ms/step, {tf:.1f} TFLOP/s", file=sys.stderr, flush=True)

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        print("# timing the CPU oracle sample", file=sys.stderr, flush=True)
        rows = np.arange(2048) if w.N > 8192 else None
        t1 = time.perf_counter()
        done, flops = 0, 0.0
        for b in range(w.B):
            for h in range(w.H):
                oracle.forward_head(f.q[b, h], f.k[b, h], f.v[b, h], w.scale, w.mask_kind, rows=rows)
                done += 1
                if rows is None:
                    flops += flop / (w.B * w.H)
                else:
                    flops += 4.0 * w.d * rows.size * (rows.size + 1) / 2
                if time.perf_counter() - t1 > args.cpu_budget:
                    break
            if time.perf_counter() - t1 > args.cpu_budget:
                break
        el = time.perf_counter() - t1
        cpu = {"value": flops / el / 1e12, "unit": "TFLOP/s", "cores": len(os.sched_getaffinity(0)), "kind": "oracle",
               "sample": f"{done} of {w.B * w.H} heads" + (", query rows 0..2047" if rows is not None else ""),
               "seconds": round(el, 2)}

    mask_name = {0: "none", 1: "causal"}[w.mask_kind]
    rec = {
        "metric": "attention fwd / fwd+bwd TFLOP/s and % of bf16 MFMA peak, N=1k-32k, d=64/128",
        "value": round(tf, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8",
        "data": "synthetic: Q, K, V ~ N(0,1) seeded, quantized to OCP E4M3 with descale 2^-4; V transposed",
        "config": {"workload": f"{w.name}: B={w.B} H={w.H} N={w.N} d={w.d} mask={mask_name} fwd, E4M3 inputs, bf16 O",
                   "B": w.B, "H": w.H, "N": w.N, "d": w.d, "mask": mask_name, "pass": "fwd", "seed": w.seed},
        "frac_of_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4),
        "roofline": {"kernel": "fwd_fp8_kernel", "bound": "mfma", "achieved": round(tf, 2),
                     "peak": round(PEAK_FP8_TFLOPS, 1), "unit": "TFLOP/s", "frac": round(tf / PEAK_FP8_TFLOPS, 4),
                     "traffic": measured_traffic(w.name, "fwd_fp8"),
                     "traffic_gbs": hbm_rate(measured_traffic(w.name, "fwd_fp8"), ms),
                     "flop_per_launch": flop, "mean_launch_ms": round(ms, 4)},
        "cpu_baseline": cpu,
        "wall_ms_per_step": round(wall * 1e3 / args.steps, 4),
    }
    print(json.dumps(rec), flush=True)
    return 0


def run_decode(args, w: synth.PackedWorkload, lens, qlens, dev) -> int:
    """Few queries per sequence against long keys: fa_fwd_splitkv per step.
    The call is two kernels (the key ranges, then the merge); both are inside
    the timed launch, whose bytes are the K and V caches read once plus Q, O
    and LSE."""
    import torch
    import io_aware_exact_10_amd as fa

    p = synth.packed_inputs(qlens, lens, w.H, w.Hkv, w.d, w.seed)

    def dev_t(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    q, k, v = dev_t(p.q_bits), dev_t(p.k_bits), dev_t(p.v_bits)
    cq, ck = torch.from_numpy(p.cu_q).to(dev), torch.from_numpy(p.cu_k).to(dev)
    Tq, Tk = q.shape[0], k.shape[0]
    mq, mk = max(qlens), max(lens)
    splits = fa.fa_splitkv_splits(w.B, w.Hkv, mk, 0)
    ws = torch.empty(fa.fa_splitkv_workspace_bytes(Tq, w.H, w.d, splits), dtype=torch.uint8, device=dev)
    o = torch.empty_like(q)
    lse = torch.empty((w.H, Tq), dtype=torch.float32, device=dev)

    def fwd():
        fa.forward_splitkv(q, k, v, cq, ck, mq, mk, w.scale, w.mask_kind, 0, out=o, lse=lse, workspace=ws)

    for _ in range(args.warmup):
        fwd()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record(stream)
        fwd()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_arr = np.array([e[0].elapsed_time(e[1]) for e in ev])
    ms = float(ms_arr.mean())
    if w.mask_kind == synth.MASK_CAUSAL:
        vis = sum(sum(max(0, min(nk, i + nk - nq + 1)) for i in range(nq)) for nq, nk in zip(qlens, lens))
    else:
        vis = sum(nq * nk for nq, nk in zip(qlens, lens))
    flop = 4.0 * w.d * vis * w.H
    copy_calibration(args.copy_calibration, dev)
    hbm_bytes = 2 * Tk * w.Hkv * w.d * 2 + 2 * Tq * w.H * w.d * 2 + Tq * w.H * 4
    gbs = hbm_bytes / (ms * 1e-3) / 1e9
    print(f"# timed {args.steps} steps: {ms:.4f} ms/step, {gbs:.0f} GB/s, splits {splits}", file=sys.stderr,
          flush=True)

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        print("# timing the CPU oracle sample", file=sys.stderr, flush=True)
        t1 = time.perf_counter()
        G = w.H // w.Hkv
        done, flops = 0, 0.0
        for b in range(w.B):
            a, e = int(p.cu_q[b]), int(p.cu_q[b + 1])
            ka, ke = int(p.cu_k[b]), int(p.cu_k[b + 1])
            for h in range(w.H):
                oracle.forward_head(p.q[a:e, h], p.k[ka:ke, h // G], p.v[ka:ke, h // G], w.scale, w.mask_kind)
                done += 1
                flops += 4.0 * w.d * (e - a) * (ke - ka)
            if time.perf_counter() - t1 > args.cpu_budget:
                break
        el = time.perf_counter() - t1
        cpu = {"value": flops / el / 1e12, "unit": "TFLOP/s", "cores": len(os.sched_getaffinity(0)),
               "kind": "oracle", "sample": f"{done} (sequence, head) pairs of {w.B * w.H}", "seconds": round(el, 2)}

    mask_name = {0: "none", 1: "causal"}[w.mask_kind]
    rec = {
        "metric": "attention fwd / fwd+bwd TFLOP/s and % of bf16 MFMA peak, N=1k-32k, d=64/128",
        "value": round(flop / (ms * 1e-3) / 1e12, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic: Q, K, V ~ N(0,1) seeded, bf16 round-to-nearest-even; key lengths uniform in [max/8, max]",
        "config": {"workload": f"{w.name}: packed B={w.B} queries/seq={w.queries} max_keys={w.max_len} "
                               f"keys={Tk} H={w.H} Hkv={w.Hkv} d={w.d} mask={mask_name} fwd (split keys)",
                   "key_lengths": lens, "H": w.H, "Hkv": w.Hkv, "d": w.d, "mask": mask_name, "pass": "fwd",
                   "splits": splits, "seed": w.seed},
        "hbm_gbs": round(gbs, 1),
        "roofline": {"kernel": "splitkv_bf16_kernel + splitkv_combine_kernel", "bound": "hbm",
                     "achieved": round(gbs, 1), "peak": 8000.0, "unit": "GB/s", "frac": round(gbs / 8000.0, 4),
                     "traffic": (None if measured_traffic(w.name, "splitkv") is None
                                 or measured_traffic(w.name, "combine") is None
                                 else measured_traffic(w.name, "splitkv") + measured_traffic(w.name, "combine")),
                     "bytes_per_launch": hbm_bytes, "mean_launch_ms": round(ms, 4)},
        "cpu_baseline": cpu,
        "wall_ms_per_step": round(wall * 1e3 / args.steps, 4),
    }
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
