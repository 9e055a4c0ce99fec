"""The seeded input generator (CPU only)."""
import numpy as np

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
