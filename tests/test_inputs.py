"""The seeded input generator: rounding is RNE with a single rounding, draws are reproducible."""
import numpy as np
import torch

import fa_inputs as FI


def test_bf16_rne_ties_and_no_double_rounding():
    one = 1.0
    cases = {
        one + 2.0 ** -8: one,                            # tie -> even (1.0)
        one + 3 * 2.0 ** -8: one + 2.0 ** -6,            # tie -> even (mantissa ...10)
        one + 2.0 ** -8 + 2.0 ** -40: one + 2.0 ** -7,   # just above the tie: up
        one + 2.0 ** -8 - 2.0 ** -40: one,               # just below the tie: down
        -(one + 2.0 ** -8 + 2.0 ** -40): -(one + 2.0 ** -7),
        (2 - 2.0 ** -8) * 2.0: 4.0,                      # carry into the exponent
        0.0: 0.0,
    }
    x = np.array(list(cases.keys()))
    got = FI.bf16_bits_to_f64(FI.f64_to_bf16_bits(x))
    assert np.array_equal(got, np.array(list(cases.values())))
    # fp64 -> fp32 -> bf16 would double-round 1 + 2^-8 + 2^-40 down to 1.0; ours must not.
    assert FI.bf16_bits_to_f64(FI.f64_to_bf16_bits(np.array([one + 2.0 ** -8 + 2.0 ** -40])))[0] != one


def test_bf16_matches_torch_on_float32_values():
    # For values already exact in float32 there is a single rounding either way.
    x32 = (np.random.Generator(np.random.PCG64(5)).standard_normal(200000) * 3).astype(np.float32)
    ours = FI.f64_to_bf16_bits(x32.astype(np.float64))
    ref = torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_bf16_subnormal_range():
    x = np.array([2.0 ** -130, 3 * 2.0 ** -134, -(2.0 ** -133) * 2.5])
    got = FI.bf16_bits_to_f64(FI.f64_to_bf16_bits(x))
    assert np.array_equal(got, np.array([2.0 ** -130, 2.0 ** -132, -(2.0 ** -132)]))


def test_fp16_rne_single_rounding():
    one = 1.0
    x = np.array([one + 2.0 ** -11, one + 3 * 2.0 ** -11, one + 2.0 ** -11 + 2.0 ** -40])
    got = FI.fp16_bits_to_f64(FI.f64_to_fp16_bits(x))
    assert np.array_equal(got, np.array([one, one + 2.0 ** -9, one + 2.0 ** -10]))


def test_draws_reproducible_and_ordered():
    a = FI.draw_bits((1, 2, 8, 4), FI.BF16, 7)
    b = FI.draw_bits((1, 2, 8, 4), FI.BF16, 7)
    for name in FI.TENSOR_ORDER:
        assert np.array_equal(a[name], b[name])
    rng = np.random.Generator(np.random.PCG64(7))
    q = rng.standard_normal((1, 2, 8, 4))
    assert np.array_equal(a["q"], FI.f64_to_bf16_bits(q))
    c = FI.draw_bits((1, 2, 8, 4), FI.BF16, 7, q_mult=4.0)
    assert np.array_equal(FI.bf16_bits_to_f64(c["q"]), 4.0 * FI.bf16_bits_to_f64(a["q"]))
    assert np.array_equal(c["k"], a["k"])


def test_workload_table():
    w = FI.WORKLOADS[FI.HEADLINE]
    assert (w.B, w.H, w.N, w.d, w.dtype, w.causal) == (4, 32, 4096, 128, FI.BF16, (True,))
    assert FI.WORKLOADS["long_context"].q_mult == 4.0


def test_draw_bits_rect_slices_draw_bits():
    # queries and keys of different lengths: the first Nq (Nk) rows of one draw over max(Nq, Nk)
    full = FI.draw_bits((2, 3, 50, 16), FI.BF16, 123)
    for nq, nk in ((50, 7), (7, 50), (50, 50)):
        r = FI.draw_bits_rect(2, 3, nq, nk, 16, FI.BF16, 123)
        assert r["q"].shape == (2, 3, nq, 16) and r["do"].shape == (2, 3, nq, 16)
        assert r["k"].shape == (2, 3, nk, 16) and r["v"].shape == (2, 3, nk, 16)
        for n, rows in (("q", nq), ("k", nk), ("v", nk), ("do", nq)):
            assert np.array_equal(r[n], full[n][:, :, :rows]) and r[n].flags["C_CONTIGUOUS"]
    a = FI.draw_bits_rect(1, 2, 5, 9, 8, FI.FP16, 7)
    b = FI.draw_bits_rect(1, 2, 5, 9, 8, FI.FP16, 7)
    assert all(np.array_equal(a[n], b[n]) for n in FI.TENSOR_ORDER)
