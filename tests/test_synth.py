"""The seeded input generator (CPU only)."""
import numpy as np
import pytest

import synth


def test_bf16_rounding_edges():
    f = np.array([1.0, -2.5, 0.0, -0.0, np.inf, -np.inf, 3.4028235e38,
                  1.0 + 2 ** -8,            # exact tie -> even (stays 1.0)
                  1.0 + 3 * 2 ** -8,        # tie -> rounds up to the even neighbour
                  1.0 + 2 ** -8 + 2 ** -20,  # above the tie -> up
                  1e-40,                    # fp32 subnormal
                  np.nan], dtype=np.float32)
    b = synth.bf16_bits(f)
    back = synth.bf16_to_f32(b)
    assert back[0] == 1.0 and back[1] == -2.5 and back[2] == 0.0
    assert np.signbit(back[3]) and back[3] == 0.0
    assert back[4] == np.inf and back[5] == -np.inf
    assert back[6] == np.inf                  # rounds past the largest finite bf16
    assert back[7] == 1.0
    assert back[8] == 1.0 + 2 ** -6
    assert back[9] == 1.0 + 2 ** -7
    assert b[10] == 0x0000 or b[10] == 0x0001  # tiny subnormal rounds to (near) zero
    assert np.isnan(back[11])


def test_bf16_matches_torch_rne():
    import torch
    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32) * 100
    ours = synth.bf16_bits(x)
    theirs = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, theirs)


def test_generator_is_deterministic_and_ordered():
    w = synth.small_workload(2, 3, 50, 64, seed=9)
    a = synth.make_inputs(w)
    b = synth.make_inputs(w)
    for x, y in ((a.q, b.q), (a.k, b.k), (a.v, b.v), (a.do, b.do)):
        assert np.array_equal(x, y)
    raw = synth.normal_tensors(9, (2, 3, 50, 64), 4)
    assert np.array_equal(a.q, synth.bf16_to_f32(synth.bf16_bits(raw[0])))
    assert np.array_equal(a.do, synth.bf16_to_f32(synth.bf16_bits(raw[3])))
    assert not np.array_equal(a.q, a.k)


def test_block_mask_density_and_diagonal():
    m = synth.block_mask(4096, 5)
    assert m.shape == (32, 32) and m.dtype == np.uint8
    assert (np.diag(m) == 1).all()
    dens = m.mean()
    assert 0.2 < dens < 0.35          # expected (32 + 0.25 * 992) / 1024 = 0.273
    big = synth.block_mask(128 * 200, 1)
    off = big[~np.eye(200, dtype=bool)]
    assert abs(off.mean() - 0.25) < 0.01


def test_workload_table():
    w = synth.WORKLOADS
    assert (w["gpt2_medium"].B, w["gpt2_medium"].H, w["gpt2_medium"].N, w["gpt2_medium"].d) == (64, 16, 1024, 64)
    assert w["long_prefill"].backward is False
    assert w["tiny_f32"].dtype == synth.DTYPE_F32
    assert abs(w["causal_train"].scale - 128 ** -0.5) < 1e-15


def test_fp8_e4m3_table_matches_the_format_definition():
    """OCP 8-bit floating point E4M3: bias 7, 3 mantissa bits, no infinities,
    S.1111.111 NaN, largest finite 448 = 1.75 * 2^8, smallest normal 2^-6,
    smallest subnormal 2^-9."""
    t = synth.fp8_e4m3_table()
    assert t[0x38] == 1.0 and t[0x7E] == 448.0 and t[0x08] == 2.0 ** -6 and t[0x01] == 2.0 ** -9
    assert t[0x07] == 7 * 2.0 ** -9 and t[0x40] == 2.0 and t[0x3F] == 1.875
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF]) and np.isnan(t).sum() == 2
    assert t[0x80] == 0.0 and np.signbit(t[0x80])
    assert (t[0x80:0xFF] == -t[0x00:0x7F]).all()
    pos = t[:0x7F]
    assert (np.diff(pos) > 0).all()                      # codes ordered by value


def test_fp8_encode_rounds_to_nearest_even():
    t = synth.fp8_e4m3_table()
    # exact values round-trip
    codes = np.array([c for c in range(256) if not np.isnan(t[c])], dtype=np.uint8)
    assert (synth.fp8_e4m3_bits(t[codes]) == codes).all()
    # midpoints go to the even code; anything else to the nearest
    for c in range(0x00, 0x7E):
        mid = (float(t[c]) + float(t[c + 1])) / 2
        assert synth.fp8_e4m3_bits(np.array([mid]))[0] == (c if c % 2 == 0 else c + 1)
        assert synth.fp8_e4m3_bits(np.array([np.nextafter(mid, 0)]))[0] == c
        assert synth.fp8_e4m3_bits(np.array([np.nextafter(mid, 1e9)]))[0] == c + 1
    assert synth.fp8_e4m3_bits(np.array([-1.0625]))[0] == 0xB8
    with pytest.raises(ValueError):
        synth.fp8_e4m3_bits(np.array([449.0]))


def test_fp8_inputs_layout():
    f = synth.fp8_inputs(2, 3, 37, 64, seed=9, pad_code=0x7F)
    assert f.ldv == 48 and f.vt8.shape == (2, 3, 64, 48)
    assert (f.vt8[..., 37:] == 0x7F).all()
    assert np.array_equal(np.swapaxes(f.vt8[..., :37], 2, 3), synth.fp8_e4m3_bits(f.v / f.v_descale))
    assert np.array_equal(f.q, synth.fp8_to_f32(f.q8) * np.float32(f.q_descale))
