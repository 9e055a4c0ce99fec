"""Host-side logic of bench.py (CPU only): the FLOP accounting against the
oracle's own visibility definition, the tile-model byte count against its
closed forms, and the counter summaries on small synthetic databases."""
import math
import sqlite3

import numpy as np
import pytest

import bench
import oracle
import synth


@pytest.mark.parametrize("mask_kind", [synth.MASK_NONE, synth.MASK_CAUSAL, synth.MASK_BLOCK_SPARSE])
@pytest.mark.parametrize("N", [1, 100, 128, 300, 513])
def test_visible_pairs_match_oracle_mask(N, mask_kind):
    """The benchmark's FLOP count uses exactly the pairs the oracle treats as visible."""
    w = synth.small_workload(1, 1, N, 64, synth.DTYPE_BF16, mask_kind, seed=11 + N)
    inp = synth.make_inputs(w)
    vis = oracle.visible(np.arange(N), N, mask_kind, inp.mask)
    assert bench.visible_pairs(w, inp.mask) == int(vis.sum())


@pytest.mark.parametrize("rows", [32, 64, 128, 256])
@pytest.mark.parametrize("N,d", [(1024, 64), (4096, 128), (640, 128)])
def test_tile_model_closed_forms(N, d, rows):
    e = 2
    nt = math.ceil(N / rows)
    full = 2 * N * d * e + nt * 2 * N * d * e + 4 * N
    assert bench.tile_model_bytes(N, d, rows, False) == full
    # causal, N a multiple of 64: query tile t reads the keys up to its last row, in 64-key tiles
    causal = 2 * N * d * e + 4 * N + sum(2 * min(N, math.ceil(min(N, (t + 1) * rows) / 64) * 64) * d * e
                                         for t in range(nt))
    assert bench.tile_model_bytes(N, d, rows, True) == causal
    assert bench.tile_model_bytes(N, d, rows, True) < full or nt == 1


def test_tile_model_falls_with_height():
    vals = [bench.tile_model_bytes(4096, 128, r, True) for r in (32, 64, 128, 256)]
    assert all(a > b for a, b in zip(vals, vals[1:]))


def _db(path, rows):
    con = sqlite3.connect(path)
    con.execute("create table counters_collection (kernel_name text, dispatch_id int, counter_name text,"
                " value real, duration real)")
    con.executemany("insert into counters_collection values (?, ?, ?, ?, ?)", rows)
    con.commit()
    con.close()


def test_traffic_summaries_scale_by_the_copy(tmp_path):
    """FETCH_SIZE / WRITE_SIZE (KiB) are scaled so that the calibration copy
    reads and writes exactly its own size; per-launch means and per-step sums."""
    copy = 1 << 30
    f, w = str(tmp_path / "f.db"), str(tmp_path / "w.db")
    k = "void fa::fwd_bf16_kernel<64, 0, 4, 2>(fa::AttnParams, unsigned int, unsigned int)"
    # the copy reads 2x its size by this counter and writes 1x; the kernel: two dispatches
    _db(f, [(bench.COPY_KERNEL, 1, "FETCH_SIZE", copy / 1024 * 2, 1.0),
            (k, 2, "FETCH_SIZE", 1000.0, 1.0), (k, 3, "FETCH_SIZE", 3000.0, 1.0)])
    _db(w, [(bench.COPY_KERNEL, 1, "WRITE_SIZE", copy / 1024, 1.0),
            (k, 2, "WRITE_SIZE", 500.0, 1.0), (k, 3, "WRITE_SIZE", 500.0, 1.0)])
    out = bench.summarize_kernel_traffic(f, w, copy, "fwd_bf16")
    row = [l for l in out.splitlines() if "fwd_bf16_kernel" in l][0]
    per_launch = (2000.0 * 1024 / 2 + 500.0 * 1024) / 1e9        # mean FETCH halved, WRITE as is
    assert float(row.split("|")[-2]) == pytest.approx(per_launch, abs=1e-3)
    step = bench.summarize_step_traffic(f, w, copy, 2)
    total = [l for l in step.splitlines() if l.startswith("Total per step")][0]
    assert f"{(4000.0 * 1024 / 2) / 2 / 1e9:.2f} GB read" in total
    assert f"{1000.0 * 1024 / 2 / 1e9:.2f} GB written" in total


def test_counter_summary_derived_columns(tmp_path):
    db = str(tmp_path / "c.db")
    k = "void fa::bwd_dq_bf16_kernel<128, 1>(fa::AttnParams, unsigned int, unsigned int)"
    cyc, ns = 1.9e6, 1.0e6                       # 1.9 GHz over 1 ms
    rows = [(k, 1, "GRBM_GUI_ACTIVE", cyc * 8, ns), (k, 1, "SQ_VALU_MFMA_BUSY_CYCLES", 0.5 * 1024 * cyc, ns),
            (k, 1, "SQ_INSTS_VALU_MFMA_MOPS_BF16", 1e9, ns)]
    _db(db, rows)
    line = [l for l in bench.summarize_counters(db).splitlines() if "bwd_dq" in l][0]
    cells = [c.strip() for c in line.split("|")]
    assert cells[4] == "1.90" and cells[5] == "0.500" and cells[6] == "512.0"


def test_stall_summary_shares(tmp_path):
    """Shares of SQ_WAVE_CYCLES from two counter passes, and instructions per MFMA."""
    a, b = str(tmp_path / "a.db"), str(tmp_path / "b.db")
    k = "void fa::fwd_bf16_kernel<128, 1, 8, 2>(fa::AttnParams, unsigned int, unsigned int)"
    _db(a, [(k, 1, "SQ_WAVE_CYCLES", 1000.0, 1.0), (k, 1, "SQ_ACTIVE_INST_ANY", 350.0, 1.0),
            (k, 1, "SQ_WAIT_ANY", 400.0, 1.0), (k, 1, "SQ_WAIT_INST_ANY", 250.0, 1.0),
            (k, 1, "SQ_ACTIVE_INST_VALU", 200.0, 1.0)])
    _db(b, [(k, 1, "SQ_INSTS_MFMA", 10.0, 1.0), (k, 1, "SQ_INSTS_VALU", 55.0, 1.0), (k, 1, "SQ_INSTS_LDS", 15.0, 1.0)])
    line = [l for l in bench.summarize_stalls([a, b]).splitlines() if "fwd_bf16" in l][0]
    cells = [c.strip() for c in line.split("|")]
    assert cells[2:7] == ["35.0 %", "40.0 %", "25.0 %", "20.0 %", "—"]
    assert cells[7:9] == ["5.50", "1.50"]


def test_pmc_summary_means_every_counter(tmp_path):
    """Per-kernel means over dispatches of each counter in the pass; kernels
    outside the library are left out."""
    db = str(tmp_path / "l.db")
    k = "void fa::bwd_dkdv8_bf16_kernel<1>(fa::AttnParams, unsigned int, unsigned int, unsigned int)"
    _db(db, [(k, 1, "LdsUtil", 30.0, 1.0), (k, 2, "LdsUtil", 36.0, 1.0),
             (k, 1, "LdsLatency", 40.0, 1.0), (k, 2, "LdsLatency", 50.0, 1.0),
             ("void other_kernel(int)", 3, "LdsUtil", 99.0, 1.0)])
    out = bench.summarize_pmc(db).splitlines()
    assert out[0] == "| kernel | dispatches | LdsUtil | LdsLatency |"
    rows = [l for l in out[2:]]
    assert len(rows) == 1
    cells = [c.strip() for c in rows[0].split("|")]
    assert cells[1:5] == ["`fa::bwd_dkdv8_bf16_kernel<1>`", "2", "33", "45"]


def test_hbm_rate():
    assert bench.hbm_rate(None, 1.0) is None
    assert bench.hbm_rate(8e9, 1.0) == 8000.0            # 8 GB in 1 ms
    assert bench.hbm_rate(541e6, 0.3445) == round(541e6 / 0.3445e-3 / 1e9, 1)


# --------------------------------------------------------------------------
# the materialise-S comparator computes attention: its O and gradients
# against the oracle, for every mask kind ("FlashAttention and IO-aware exact
# attention", "How to approach it": the naive and the blockwise result on the
# same random inputs)
# --------------------------------------------------------------------------
@pytest.mark.parametrize("mask_kind", [synth.MASK_NONE, synth.MASK_CAUSAL, synth.MASK_BLOCK_SPARSE])
@pytest.mark.parametrize("dtype", ["f64", "bf16"])
def test_naive_comparator_matches_oracle(mask_kind, dtype):
    import torch
    w = synth.small_workload(2, 3, 300, 16, synth.DTYPE_BF16, mask_kind, seed=61)
    inp = synth.make_inputs(w)
    tdt = torch.float64 if dtype == "f64" else torch.bfloat16
    # inp.q etc. hold the bf16-rounded values; both dtypes see exactly them
    q, k, v, do = (torch.from_numpy(np.ascontiguousarray(a)).to(tdt) for a in (inp.q, inp.k, inp.v, inp.do))
    mask_t = torch.from_numpy(inp.mask) if inp.mask is not None else None
    bm = bench.naive_mask(w, mask_t, torch.device("cpu"))
    o, grads = bench.naive_step(q, k, v, do, w.scale, w.mask_kind, bm, True)
    O, _ = oracle.forward(inp.q, inp.k, inp.v, w.scale, w.mask_kind, inp.mask)
    ref = (O,) + oracle.backward(inp.q, inp.k, inp.v, inp.do, w.scale, w.mask_kind, inp.mask)
    got = [t.double().numpy().reshape(r.shape) for t, r in zip((o,) + grads, ref)]
    # f64: the comparator keeps its softmax in fp32 (P is rounded there);
    # bf16: the bf16 tolerances the kernels meet (O 2e-2, gradients 5e-2 max-normalised)
    o_tol, g_tol = (1e-5, 1e-5) if dtype == "f64" else (2e-2, 5e-2)
    assert np.abs(got[0] - ref[0]).max() <= o_tol
    for g, r in zip(got[1:], ref[1:]):
        assert np.abs(g - r).max() / max(np.abs(r).max(), 1e-3) <= g_tol
    # the comparator materialises the full N x N score matrix of each head
    assert bm is None or tuple(bm.shape) == (w.N, w.N)


@pytest.mark.parametrize("mask_kind", [synth.MASK_NONE, synth.MASK_CAUSAL, synth.MASK_BLOCK_SPARSE])
def test_visible_pairs_of_a_row_sample_match_oracle_mask(mask_kind):
    """The CPU baseline credits the oracle with the visible pairs of exactly
    the rows it samples."""
    N = 700
    w = synth.small_workload(1, 1, N, 64, synth.DTYPE_BF16, mask_kind, seed=71)
    inp = synth.make_inputs(w)
    rows = np.arange(0, N, 7)
    vis = oracle.visible(rows, N, mask_kind, inp.mask)
    assert bench.visible_pairs_rows(w, inp.mask, rows) == int(vis.sum())


def test_source_digest_ignores_comments_only(tmp_path):
    """A counter record stays valid across comment edits and goes stale on code edits."""
    a, b, c = tmp_path / "a.hip", tmp_path / "b.hip", tmp_path / "c.hip"
    a.write_text("// header\nint f(int x) { return x + 1; }  /* note */\n")
    b.write_text("// another header\n/* block\n comment */\nint f(int x) {\n  return x + 1;  // tail\n}\n")
    c.write_text("// header\nint f(int x) { return x + 2; }\n")
    assert bench.source_digest(str(a)) == bench.source_digest(str(b))
    assert bench.source_digest(str(a)) != bench.source_digest(str(c))
