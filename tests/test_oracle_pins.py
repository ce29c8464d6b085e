"""Pins for the CPU oracle: each check ties it to something other than itself
(values printed on the pages, IEEE 754 facts, a library routine for a special
case, brute force, exact rational arithmetic)."""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import w4a16_ref as ref

# ---------------------------------------------------------------------------
# 16-bit conversions
# ---------------------------------------------------------------------------


def _all_finite_f16():
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    f = b.view(np.float16)
    return b[np.isfinite(f)]


def test_f16_widening_matches_numpy_for_every_pattern():
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = ref.f16_bits_to_f64(b)
    lib = b.view(np.float16).astype(np.float64)
    nan = np.isnan(lib)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], lib[~nan])


def test_f16_narrowing_roundtrips_every_finite_value():
    b = _all_finite_f16()
    f32 = b.view(np.float16).astype(np.float32)
    assert np.array_equal(ref.f32_to_f16_bits(f32), b)


def test_f16_narrowing_midpoints_and_neighbours_match_numpy():
    # midpoints between consecutive non-negative finite fp16 values are exact in fp32
    b = np.arange(0, 0x7C00, dtype=np.uint32).astype(np.uint16)
    lo = b.view(np.float16).astype(np.float64)
    hi = (b + 1).astype(np.uint16).view(np.float16).astype(np.float64)
    hi[-1] = 65520.0  # the rounding boundary above the largest finite value
    mid = ((lo + hi) / 2).astype(np.float32)
    cases = [mid, np.nextafter(mid, np.float32(np.inf)), np.nextafter(mid, np.float32(0))]
    x = np.concatenate(cases)
    x = np.concatenate([x, -x])
    assert np.array_equal(ref.f32_to_f16_bits(x), x.astype(np.float16).view(np.uint16))


def test_f16_narrowing_random_patterns_match_numpy():
    rng = np.random.default_rng(7)
    u = rng.integers(0, 2**32, size=2_000_000, dtype=np.uint64).astype(np.uint32)
    x = u.view(np.float32)
    x = x[~np.isnan(x)]
    with np.errstate(over="ignore"):
        lib = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(ref.f32_to_f16_bits(x), lib)


def test_f16_ieee_special_cases():
    # closed forms from the binary16 definition
    cases = [
        (0.0, 0x0000), (-0.0, 0x8000), (1.0, 0x3C00), (-2.0, 0xC000),
        (65504.0, 0x7BFF), (65519.0, 0x7BFF), (65520.0, 0x7C00), (1e9, 0x7C00),
        (2.0**-24, 0x0001), (2.0**-25, 0x0000),            # tie -> even (zero)
        (3 * 2.0**-25, 0x0002),                            # tie between 1 and 2 units -> 2
        (2.0**-14, 0x0400), (1.0 + 2.0**-11, 0x3C00),      # tie -> even
        (1.0 + 3 * 2.0**-11, 0x3C02), (float("inf"), 0x7C00), (float("-inf"), 0xFC00),
    ]
    for v, bits in cases:
        assert int(ref.f32_to_f16_bits(np.array([v], np.float32))[0]) == bits, v
    assert int(ref.f32_to_f16_bits(np.array([np.nan], np.float32))[0]) & 0x7C00 == 0x7C00


def test_bf16_narrowing_matches_torch():
    rng = np.random.default_rng(11)
    u = rng.integers(0, 2**32, size=2_000_000, dtype=np.uint64).astype(np.uint32)
    x = u.view(np.float32)
    x = x[~np.isnan(x)]
    lib = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ref.f32_to_bf16_bits(x), lib)
    # exact ties
    t = (np.arange(1, 1 << 16, dtype=np.uint32) << 16) | np.uint32(0x8000)
    t = t[((t >> 23) & 0xFF) != 0xFF].view(np.float32)
    lib = torch.from_numpy(t).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ref.f32_to_bf16_bits(t), lib)


def test_bf16_widening_every_pattern():
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = ref.bf16_bits_to_f64(b)
    lib = torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).double().numpy()
    nan = np.isnan(lib)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], lib[~nan])


# ---------------------------------------------------------------------------
# Byte accounting: values printed on the pages
# ---------------------------------------------------------------------------


def test_sizing_matches_printed_values(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "memory_arithmetic.json")))
    bpw = ref.bits_per_weight(128)
    assert bpw == 4.15625
    assert round(bpw, 3) == g["bits_per_weight_g128_printed"]
    n13 = g["params_13b"]
    assert ref.model_bytes(n13, 16) / 1e9 == g["fp16_weight_bytes_13b_printed_GB"]
    assert round(ref.model_bytes(n13, bpw) / 1e9, 2) == g["w4_weight_bytes_13b_printed_GB"]
    assert round(ref.model_bytes(n13, g["bits_per_weight_g128_printed"]) / 1e9, 2) == \
        g["w4_weight_bytes_13b_printed_GB"]
    saved = ref.model_bytes(n13, 16) - ref.model_bytes(n13, bpw)
    assert round(saved / 1e9, 1) == g["saved_13b_printed_GB"]
    assert round(g["hidden_13b"] * 2 / 1e3, 1) == g["one_token_activation_fp16_printed_kB"]
    assert round(g["hidden_13b"] * 1 / 1e3, 1) == g["one_token_activation_int8_printed_kB"]
    n70 = g["params_70b"]
    assert ref.model_bytes(n70, 16) / 1e9 == g["bf16_weight_bytes_70b_printed_GB"]
    assert ref.model_bytes(n70, 4) / 1e9 == g["int4_weight_bytes_70b_printed_GB"]


@pytest.mark.parametrize("N,K,group", [(4096, 4096, 128), (8192, 28672, 32), (5120, 13824, 128),
                                       (15360, 5120, 64)])
def test_packed_bytes_equal_bits_per_weight(N, K, group):
    q, s, z = ref.packed_bytes(N, K, group)
    assert (q + s + z) * 8 == N * K * ref.bits_per_weight(group)
    assert q * 8 == 4 * N * K


# ---------------------------------------------------------------------------
# Quantiser
# ---------------------------------------------------------------------------


def _exact_w_hat(codes, s_bits, zeros, group):
    return ref.dequantize(codes, s_bits, zeros, group)


@pytest.mark.parametrize("group", [32, 64, 128])
def test_quantizer_codes_are_nearest_grid_points(group):
    rng = np.random.default_rng(group)
    w = (rng.standard_normal((24, 4 * group)) * 0.02).astype(np.float32)
    w[3] = np.abs(w[3])          # one-signed rows
    w[4] = -np.abs(w[4])
    w[5, :group] = 0.25          # constant group
    codes, s_bits, zeros = ref.quantize_groupwise(w, group)
    N, K = w.shape
    G = K // group
    s = ref.f16_bits_to_f64(s_bits).T                     # [N][G]
    z = zeros.T.astype(np.int64)
    w64 = w.astype(np.float64).reshape(N, G, group)
    grid = (np.arange(16)[None, None, None, :] - z[:, :, None, None]) * s[:, :, None, None]
    dist = np.abs(w64[..., None] - grid)                  # [N][G][g][16]
    best = dist.min(axis=-1)
    got = np.take_along_axis(dist, codes.reshape(N, G, group, 1).astype(np.int64), axis=-1)[..., 0]
    assert np.all(got <= best + 2.0**-20 * np.abs(w64) + 1e-30)


def test_quantizer_exact_ties_round_to_even():
    s = 2.0**-6
    j = np.arange(-8, 7)                           # (j + 1/2) s lies strictly inside the grid
    vals = np.concatenate([[-8 * s, 7 * s], (j + 0.5) * s, np.zeros(128 - 2 - j.size)])
    w = vals.astype(np.float32)[None, :]
    codes, s_bits, zeros = ref.quantize_groupwise(w, 128)
    assert ref.f16_bits_to_f64(s_bits)[0, 0] == s
    assert zeros[0, 0] == 8
    d = codes[0, 2:2 + j.size].astype(np.int64) - 8
    want = np.where(j % 2 == 0, j, j + 1)          # the even one of j, j+1
    assert np.array_equal(d, want)


@pytest.mark.parametrize("group", [32, 64, 128])
def test_round_trip_error_within_half_scale(group):
    rng = np.random.default_rng(100 + group)
    w = (rng.standard_t(4, size=(64, 8 * group)) * 0.02).astype(np.float32)
    codes, s_bits, zeros = ref.quantize_groupwise(w, group)
    w_hat = _exact_w_hat(codes, s_bits, zeros, group)
    N, K = w.shape
    G = K // group
    s = np.repeat(ref.f16_bits_to_f64(s_bits).T, group, axis=1)
    err = np.abs(w.astype(np.float64) - w_hat)
    inner = (codes > 0) & (codes < 15)
    assert np.all(err[inner] <= 0.5 * s[inner] + 2.0**-24 * np.abs(w[inner]))
    # clamped codes: half a step plus the fp16 rounding of the scale over 15 steps
    wg = w.astype(np.float64).reshape(N, G, group)
    s_real = (np.maximum(wg.max(2), 0) - np.minimum(wg.min(2), 0)) / 15
    s_real = np.repeat(s_real, group, axis=1)
    bound = 0.5 * s + 15 * np.abs(s_real - s) + 2.0**-20 * np.abs(w).max()
    assert np.all(err <= bound)


@pytest.mark.parametrize("group", [32, 64, 128])
def test_lattice_weights_are_reproduced_exactly(group):
    rng = np.random.default_rng(200 + group)
    N, G = 40, 6
    q = rng.integers(0, 16, size=(N, G, group))
    q[:, :, 0] = 0
    q[:, :, 1] = 15
    q = np.take_along_axis(q, rng.permuted(np.tile(np.arange(group), (N, G, 1)), axis=2), axis=2)
    z = rng.integers(0, 16, size=(N, G))
    e = rng.integers(-20, -2, size=(N, G))
    s = np.ldexp(1.0, e)
    W = ((q - z[:, :, None]) * s[:, :, None]).reshape(N, G * group).astype(np.float32)
    codes, s_bits, zeros = ref.quantize_groupwise(W, group)
    assert np.array_equal(codes.reshape(N, G, group), q.astype(np.uint8))
    assert np.array_equal(ref.f16_bits_to_f64(s_bits).T, s)
    assert np.array_equal(zeros.T, z.astype(np.uint8))
    assert np.array_equal(_exact_w_hat(codes, s_bits, zeros, group), W.astype(np.float64))


def test_degenerate_groups():
    w = np.zeros((8, 96), dtype=np.float32)
    w[1, :32] = 1e-12                                    # range underflows fp16
    w[2, :32] = 0.5                                      # constant positive group
    w[3, :32] = -0.5                                     # constant negative group
    codes, s_bits, zeros = ref.quantize_groupwise(w, 32)
    assert s_bits[0, 0] == 0x0001 and zeros[0, 0] == 0 and codes[0, 0] == 0
    assert s_bits[0, 1] == 0x0001 and np.all(codes[1, :32] == 0)
    w_hat = ref.dequantize(codes, s_bits, zeros, 32)
    assert np.all(w_hat[0] == 0.0)
    assert np.all(w_hat[4:] == 0.0)
    assert zeros[0, 2] == 0 and np.all(codes[2, :32] == 15)
    assert zeros[0, 3] == 15 and np.all(codes[3, :32] == 0)
    s2 = ref.f16_bits_to_f64(s_bits[0, 2])
    assert abs(w_hat[2, 0] - 0.5) <= 15 * abs(0.5 / 15 - s2) + 1e-12


def test_quantizer_rejects_bad_input():
    with pytest.raises(ValueError):
        ref.quantize_groupwise(np.zeros((8, 100), np.float32), 32)
    with pytest.raises(ValueError):
        ref.quantize_groupwise(np.full((8, 32), np.inf, np.float32), 32)


# ---------------------------------------------------------------------------
# Dequantisation and product
# ---------------------------------------------------------------------------


def _frac_f16(bits):
    v = ref.f16_bits_to_f64(np.uint16(bits))
    return Fraction(float(v))


@pytest.mark.parametrize("M,N,K,group,dtype", [(1, 8, 32, 32, "f16"), (3, 16, 256, 64, "f16"),
                                               (2, 16, 128, 128, "bf16")])
def test_product_matches_exact_rational_sum(M, N, K, group, dtype):
    rng = np.random.default_rng(M * 1000 + N + K)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    x32 = rng.standard_normal((M, K)).astype(np.float32)
    xb = x32.astype(np.float16).view(np.uint16) if dtype == "f16" else \
        torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    codes, s_bits, zeros = ref.quantize_groupwise(w, group)
    y, a = ref.linear_ref_rows(xb, dtype, codes, s_bits, zeros, group)
    xv = ref.act_bits_to_f64(xb, dtype)
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            acc_abs = Fraction(0)
            for k in range(K):
                g = k // group
                wk = _frac_f16(s_bits[g, n]) * (int(codes[n, k]) - int(zeros[g, n]))
                term = Fraction(float(xv[m, k])) * wk
                acc += term
                acc_abs += abs(term)
            assert abs(Fraction(float(y[m, n])) - acc) <= K * Fraction(2) ** -53 * acc_abs
            assert abs(Fraction(float(a[m, n])) - acc_abs) <= K * Fraction(2) ** -53 * acc_abs


def test_one_hot_activation_selects_a_dequantised_weight():
    rng = np.random.default_rng(5)
    w = (rng.standard_normal((16, 128)) * 0.02).astype(np.float32)
    codes, s_bits, zeros = ref.quantize_groupwise(w, 64)
    w_hat = ref.dequantize(codes, s_bits, zeros, 64)
    for k in (0, 63, 64, 127):
        x = np.zeros((1, 128), dtype=np.float16)
        x[0, k] = 1.0
        y, a = ref.linear_ref(x.view(np.uint16), "f16", w_hat)
        assert np.array_equal(y[0], w_hat[:, k])
        assert np.array_equal(a[0], np.abs(w_hat[:, k]))


def test_error_ratio_bar():
    y_ref = np.array([[1.0, 0.0]])
    a = np.array([[10.0, 0.0]])
    r = ref.error_ratio(np.array([[1.0 + 0.02001, 1e-5]]), y_ref, a)
    assert np.allclose(r, [[1.0, 1.0]], rtol=1e-9)
    # fp16 outputs are held to the bare bar; bf16 outputs get half a bf16 ulp at |y|
    r16 = ref.error_ratio(np.array([[1.0 + 0.02001]]), np.array([[1.0]]), np.array([[10.0]]), "f16")
    rbf = ref.error_ratio(np.array([[1.0 + 0.02001 + 2.0 ** -8]]), np.array([[1.0]]), np.array([[10.0]]), "bf16")
    assert np.allclose(r16, 1.0, rtol=1e-6) and np.allclose(rbf, 1.0, rtol=1e-6)


def test_correctly_rounded_fp16_always_meets_the_bare_bar():
    """For every positive finite fp16 value v (subnormals included), the exact
    results farthest from v that still round to it (v minus and plus half the
    gaps to its neighbours), at the tightest budget sum|x*w_hat| = |y|: the
    rounding alone stays within a quarter of the bare bar, so fp16 needs no
    rounding term."""
    bits = np.arange(1, 0x7BFF, dtype=np.uint16)
    v = bits.view(np.float16).astype(np.float64)
    up = np.spacing(bits.view(np.float16)).astype(np.float64) / 2
    down = (v - (bits - 1).view(np.float16).astype(np.float64)) / 2
    worst = 0.0
    for y in (v + up, v - down):   # rounding error half a gap either way
        r = ref.error_ratio(v, y, np.abs(y), "f16")
        worst = max(worst, float(r.max()))
    assert worst <= 2.0 ** -11 / 2e-3 + 1e-12 and worst < 0.25
    # and on random fp64 results rounded by numpy (round to nearest even)
    rng = np.random.default_rng(3)
    y = rng.standard_normal(200000) * np.exp2(rng.integers(-26, 15, 200000))
    r = ref.error_ratio(y.astype(np.float16).astype(np.float64), y, np.abs(y), "f16")
    assert float(r.max()) < 0.25


def test_linear_ref_rows_columns_equal_the_full_product():
    """linear_ref_rows(cols=...) gives exactly the columns `cols` of
    linear_ref over the whole dequantised matrix (same fp64 products)."""
    rng = np.random.default_rng(12)
    N, K, group, M = 48, 256, 32, 5
    w = rng.standard_normal((N, K)).astype(np.float32)
    codes, s_bits, zeros = ref.quantize_groupwise(w, group)
    x = ref.f32_to_f16_bits(rng.standard_normal((M, K)).astype(np.float32))
    y_all, a_all = ref.linear_ref(x, "f16", ref.dequantize(codes, s_bits, zeros, group))
    for cols in (np.array([0]), np.array([N - 1, 3, 17]), np.arange(0, N, 5)):
        y, a = ref.linear_ref_rows(x, "f16", codes, s_bits, zeros, group, cols)
        assert np.array_equal(y, y_all[:, cols]) and np.array_equal(a, a_all[:, cols])
    y, a = ref.linear_ref_rows(x, "f16", codes, s_bits, zeros, group)
    assert np.array_equal(y, y_all) and np.array_equal(a, a_all)


def test_out_half_ulp_fp16_matches_numpy_spacing():
    """Half the fp16 spacing at every positive finite fp16 value below the
    largest (subnormals included)."""
    v = np.arange(1, 0x7BFF, dtype=np.uint16).view(np.float16)
    want = np.spacing(v).astype(np.float64) / 2
    assert np.array_equal(ref.out_half_ulp(v.astype(np.float64), "f16"), want)
    assert ref.out_half_ulp(0.0, "f16") == 2.0 ** -25


def test_out_half_ulp_bf16_is_half_the_gap_to_the_next_value():
    """bf16: half the distance from a value to its successor (bit pattern + 1), for
    every positive finite bf16 value below the largest."""
    bits = np.arange(1, 0x7F7F, dtype=np.uint32).astype(np.uint16)
    v = ref.bf16_bits_to_f64(bits)
    gap = ref.bf16_bits_to_f64((bits + 1).astype(np.uint16)) - v
    assert np.array_equal(ref.out_half_ulp(v, "bf16"), gap / 2)


def test_exactly_rounded_bf16_result_needs_the_rounding_term():
    """A short-K product whose |y| is close to sum|x*w_hat|: the exact result
    rounded once to bf16 is off the 2e-3 bar on its own, inside it once the
    rounding is counted."""
    x = np.array([[1.0, 1.0]], dtype=np.float64)
    w_hat = np.array([[0.5, 0.50390625 + 2.0 ** -10]])      # y = A, just past a bf16 midpoint
    y = x @ w_hat.T
    a = np.abs(x) @ np.abs(w_hat).T
    y_bf = ref.bf16_bits_to_f64(ref.f32_to_bf16_bits(y.astype(np.float32)))
    assert ref.error_ratio(y_bf, y, a)[0, 0] > 1.0
    assert ref.error_ratio(y_bf, y, a, "bf16")[0, 0] <= 1.0


# ---------------------------------------------------------------------------
# Layouts
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("N,K", [(64, 32), (72, 64), (200, 96), (8, 32), (136, 256)])
def test_device_layout_is_a_permutation(N, K):
    idx = ref._device_nibble_index(N, K).ravel()
    assert np.array_equal(np.sort(idx), np.arange(N * K))


def test_device_layout_worked_example(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "device_layout_example.json")))
    N, K = g["N"], g["K"]
    for p in g["positions"]:
        codes = np.zeros((N, K), dtype=np.uint8)
        codes[p["n"], p["k"]] = 0xA
        packed = ref.pack_device(codes)
        nz = np.nonzero(packed)[0]
        assert list(nz) == [p["byte"]], p
        assert packed[p["byte"]] == (0xA0 if p["high_nibble"] else 0x0A), p


@pytest.mark.parametrize("N,K", [(72, 64), (200, 96), (4096, 128)])
def test_device_layout_round_trip(N, K):
    rng = np.random.default_rng(N + K)
    codes = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
    packed = ref.pack_device(codes)
    assert packed.size == N * K // 2
    assert np.array_equal(ref.unpack_device(packed, N, K), codes)


def test_zero_packing_by_hand():
    z = np.array([[1, 2, 3, 4, 5, 6, 7, 8, 15, 0, 0, 0, 0, 0, 0, 9]], dtype=np.uint8)
    words = ref.pack_zeros(z)
    assert words.tolist() == [[0x87654321, 0x9000000F]]
    assert np.array_equal(ref.unpack_zeros(words, 1, 16), z)


def test_device_metadata_layout_by_hand():
    # row-major metadata, each row padded to a multiple of 8 groups:
    # group 32, N = 8 rows, K = 160 -> G = 5 groups, G8 = 8 slots per row
    G, N = 5, 8
    s_bits = (np.arange(G * N, dtype=np.uint16).reshape(G, N) + 1)   # s_bits[g, n] = 1 + 8 g + n
    z = (np.arange(G * N, dtype=np.uint8).reshape(G, N) % 16)         # z[g, n] = (8 g + n) % 16
    ds = ref.pack_scales_device(s_bits, 32)
    assert ds.shape == (8, 8)
    # row 3: groups 0..4 are 1 + 3, 9 + 3, 17 + 3, 25 + 3, 33 + 3, then three padded zeros
    assert ds[3].tolist() == [4, 12, 20, 28, 36, 0, 0, 0]
    assert ds[7].tolist() == [8, 16, 24, 32, 40, 0, 0, 0]
    dz = ref.pack_zeros_device(z, 32)
    assert dz.shape == (8, 1)
    # row 2: z = 2, 10, 18 % 16 = 2, 26 % 16 = 10, 34 % 16 = 2 in nibbles 0..4
    assert int(dz[2, 0]) == 0x0002A2A2
    # row 7: 7, 15, 23 % 16 = 7, 31 % 16 = 15, 39 % 16 = 7
    assert int(dz[7, 0]) == 0x0007F7F7
    assert ref.device_meta_bytes(8, 160, 32) == (2 * 8 * 8, 8 * 8 // 2)
    # group 128, K = 1280 -> G = 10 groups, G8 = 16: row n's 16 slots start at 32 n bytes
    s10 = np.arange(10 * 16, dtype=np.uint16).reshape(10, 16)
    d10 = ref.pack_scales_device(s10, 128)
    assert d10.shape == (16, 16) and d10[5, 9] == s10[9, 5] and d10[5, 10] == 0
    z10 = (np.arange(10 * 16, dtype=np.uint8).reshape(10, 16) % 16)
    w10 = ref.pack_zeros_device(z10, 128)
    assert w10.shape == (16, 2)
    # row 1, groups 8 and 9 (z = (16 g + 1) % 16 = 1) in nibbles 0 and 1 of word 1
    assert int(w10[1, 1]) == 0x00000011
    assert ref.device_meta_bytes(16, 1280, 128) == (2 * 16 * 16, 16 * 16 // 2)


# ---------------------------------------------------------------------------
# Symmetric formats (sym4, sym8 = W8A16) and group 256
# ---------------------------------------------------------------------------

SYM = [("sym4", 7), ("sym8", 127)]


@pytest.mark.parametrize("fmt,qmax", SYM)
@pytest.mark.parametrize("group", [32, 128, 256])
def test_symmetric_codes_are_nearest_signed_grid_points(fmt, qmax, group):
    """Brute force over every signed code: the chosen one is a nearest grid
    point q*s, q in [-qmax-1, qmax]; the zero is the fixed offset qmax+1."""
    rng = np.random.default_rng(qmax + group)
    w = (rng.standard_t(5, size=(12, 2 * group)) * 0.03).astype(np.float32)
    w[2] = np.abs(w[2])
    w[3, :group] = -0.125
    codes, s_bits, zeros = ref.quantize_groupwise(w, group, fmt)
    N, K = w.shape
    G = K // group
    assert np.all(zeros == qmax + 1)
    s = ref.f16_bits_to_f64(s_bits).T
    # the scale: max|w| / qmax in fp32, rounded to fp16 (checked through numpy's own fp16)
    amax = np.abs(w.reshape(N, G, group)).max(2)
    want_s = (amax / np.float32(qmax)).astype(np.float16).astype(np.float64)
    assert np.array_equal(s, want_s)
    grid = np.arange(-qmax - 1, qmax + 1)[None, None, None, :] * s[:, :, None, None]
    w64 = w.astype(np.float64).reshape(N, G, group)
    dist = np.abs(w64[..., None] - grid)
    got = np.take_along_axis(dist, codes.reshape(N, G, group, 1).astype(np.int64), axis=-1)[..., 0]
    assert np.all(got <= dist.min(-1) + 2.0 ** -20 * np.abs(w64) + 1e-30)
    # nothing reaches the clamp: |w| <= max|w| ~ qmax * s
    assert codes.min() >= 1


@pytest.mark.parametrize("fmt,qmax", SYM)
def test_symmetric_is_odd(fmt, qmax):
    """Round half to even is odd-symmetric and the range is |w|: negating the
    weights negates the rebuilt weights exactly."""
    rng = np.random.default_rng(7)
    w = (rng.standard_normal((16, 512)) * 0.05).astype(np.float32)
    a = ref.dequantize(*ref.quantize_groupwise(w, 64, fmt), 64)
    b = ref.dequantize(*ref.quantize_groupwise(-w, 64, fmt), 64)
    assert np.array_equal(a, -b)


@pytest.mark.parametrize("fmt,qmax", SYM)
def test_symmetric_ties_round_to_even(fmt, qmax):
    s = 2.0 ** -5
    j = np.arange(-qmax, qmax)                     # (j + 1/2) s strictly inside [-qmax, qmax] s
    vals = np.concatenate([[qmax * s], (j + 0.5) * s])
    K = 256
    vals = np.concatenate([vals, np.zeros(-vals.size % K)]) if vals.size <= K else vals
    w = vals.astype(np.float32)[None, :]
    w = np.tile(w, (8, 1))
    group = w.shape[1] if w.shape[1] in (32, 64, 128, 256) else 256
    codes, s_bits, zeros = ref.quantize_groupwise(w, group, fmt)
    assert ref.f16_bits_to_f64(s_bits)[0, 0] == s
    d = codes[0, 1:1 + j.size].astype(np.int64) - (qmax + 1)
    assert np.array_equal(d, np.where(j % 2 == 0, j, j + 1))


@pytest.mark.parametrize("fmt,qmax", SYM)
@pytest.mark.parametrize("group", [32, 256])
def test_symmetric_lattice_weights_are_reproduced_exactly(fmt, qmax, group):
    rng = np.random.default_rng(300 + qmax + group)
    N, G = 24, 3
    q = rng.integers(-qmax, qmax + 1, size=(N, G, group))
    q[:, :, 0] = np.where(rng.random((N, G)) < 0.5, qmax, -qmax)     # |q| = qmax present
    e = rng.integers(-18, -3, size=(N, G))
    s = np.ldexp(1.0, e)
    W = (q * s[:, :, None]).reshape(N, G * group).astype(np.float32)
    codes, s_bits, zeros = ref.quantize_groupwise(W, group, fmt)
    assert np.array_equal(codes.reshape(N, G, group).astype(np.int64) - (qmax + 1), q)
    assert np.array_equal(ref.f16_bits_to_f64(s_bits).T, s)
    assert np.array_equal(ref.dequantize(codes, s_bits, zeros, group), W.astype(np.float64))


@pytest.mark.parametrize("fmt,qmax", SYM)
def test_symmetric_round_trip_within_half_scale(fmt, qmax):
    rng = np.random.default_rng(11)
    w = (rng.standard_normal((32, 1024)) * 0.02).astype(np.float32)
    codes, s_bits, zeros = ref.quantize_groupwise(w, 128, fmt)
    err = np.abs(w.astype(np.float64) - ref.dequantize(codes, s_bits, zeros, 128))
    s = np.repeat(ref.f16_bits_to_f64(s_bits).T, 128, axis=1)
    assert np.all(err <= 0.5 * s + 2.0 ** -24 * np.abs(w))


def test_symmetric_degenerate_groups():
    w = np.zeros((8, 64), dtype=np.float32)
    w[1, :32] = 1e-12
    w[2, :32] = -0.5
    for fmt, qmax in SYM:
        codes, s_bits, zeros = ref.quantize_groupwise(w, 32, fmt)
        assert s_bits[0, 0] == 0x0001 and np.all(codes[0] == qmax + 1)    # all-zero group: q = 0
        assert s_bits[0, 1] == 0x0001 and np.all(codes[1, :32] == qmax + 1)
        assert np.all(codes[2, :32] == 1)                                  # -max|w| -> -qmax
        w_hat = ref.dequantize(codes, s_bits, zeros, 32)
        assert np.all(w_hat[0] == 0.0) and np.all(w_hat[1] == 0.0)


def test_int8_per_tensor_matches_integer_search():
    """The pages' per-tensor symmetric INT8 (one group spanning a row here):
    every code is the integer nearest to w/s, found by a search over all 256."""
    rng = np.random.default_rng(5)
    w = rng.standard_normal((4, 256)).astype(np.float32)
    codes, s_bits, zeros = ref.quantize_groupwise(w, 256, "sym8")
    s = ref.f16_bits_to_f64(s_bits)[0]
    for n in range(4):
        cand = np.arange(-128, 128)
        best = cand[np.argmin(np.abs(w[n][:, None].astype(np.float64) - cand[None, :] * s[n]), axis=1)]
        assert np.array_equal(codes[n].astype(np.int64) - 128, best)


def test_format_byte_accounting():
    for N, K, g in [(4096, 4096, 128), (5120, 13824, 256), (8192, 28672, 32)]:
        for fmt in ("asym4", "sym4", "sym8"):
            q, s, z = ref.packed_bytes(N, K, g, fmt)
            assert (q + s + z) * 8 == N * K * ref.format_bits_per_weight(g, fmt)
    assert ref.format_bits_per_weight(128, "asym4") == 4.15625
    assert ref.format_bits_per_weight(128, "sym4") == 4.125
    assert ref.format_bits_per_weight(256, "sym8") == 8.0625
    assert ref.format_bits_per_weight(256, "asym4") == 4 + 20 / 256
    assert ref.packed_bytes(64, 512, 256, "sym8") == (64 * 512, 2 * 2 * 64, 0)
    assert ref.device_meta_bytes(64, 512, 256, "sym4") == (2 * 8 * 64, 0)


def test_group256_metadata_layout():
    G, N = 3, 16
    s_bits = np.arange(1, G * N + 1, dtype=np.uint16).reshape(G, N)
    z = (np.arange(G * N, dtype=np.uint8).reshape(G, N) * 5) % 16
    ds = ref.pack_scales_device(s_bits, 256)
    assert ds.shape == (N, 8)
    assert np.array_equal(ds[:, :G], s_bits.T) and not ds[:, G:].any()
    dz = ref.pack_zeros_device(z, 256)
    # row 4: z = (5 * (16 g + 4)) % 16 = 4 for g = 0, 1, 2
    assert dz.shape == (N, 1) and int(dz[4, 0]) == 0x444
    assert ref.device_meta_bytes(N, 768, 256) == (2 * 8 * N, 8 * N // 2)


def test_group256_groups_span_two_columns():
    """A group of 256 straddles two 128-weight columns: its range and scale come
    from both halves (a group-128 quantisation of the same row differs)."""
    w = np.zeros((8, 256), dtype=np.float32)
    w[:, :128] = 0.01
    w[:, 128:] = -1.5
    c256, s256, z256 = ref.quantize_groupwise(w, 256)
    c128, s128, z128 = ref.quantize_groupwise(w, 128)
    assert s256.shape == (1, 8) and s128.shape == (2, 8)
    assert ref.f16_bits_to_f64(s256[0, 0]) == ref.f16_bits_to_f64(ref.f32_to_f16_bits(np.float32(1.51) / np.float32(15)))
    lo, hi = -1.5, 0.01
    s = float(ref.f16_bits_to_f64(s256[0, 0]))
    assert z256[0, 0] == int(np.clip(np.rint(np.float32(-lo) / np.float32(s)), 0, 15))
    # the small half is lost inside the wide group (w_hat = 0), kept at group 128
    w_hat256 = ref.dequantize(c256, s256, z256, 256)
    w_hat128 = ref.dequantize(c128, s128, z128, 128)
    assert np.all(w_hat256[:, :128] == 0.0)
    assert np.all(np.abs(w_hat128[:, :128] - 0.01) < 1e-5)


@pytest.mark.parametrize("N,K", [(72, 64), (200, 96), (16, 256)])
def test_sym8_planes_round_trip_and_order(N, K):
    rng = np.random.default_rng(N * K)
    codes = rng.integers(0, 256, size=(N, K), dtype=np.uint8)
    packed = ref.pack_device(codes, "sym8")
    assert packed.size == N * K
    assert np.array_equal(ref.unpack_device(packed, N, K, "sym8"), codes)
    # plane 0 is the 4-bit layout of the low nibbles, plane 1 of the high nibbles
    assert np.array_equal(packed[:N * K // 2], ref.pack_device(codes & 0xF))
    one = np.zeros((N, K), dtype=np.uint8)
    one[N - 1, K - 1] = 0xA5
    p1 = ref.pack_device(one, "sym8")
    nz = np.nonzero(p1)[0]
    assert len(nz) == 2 and nz[1] - nz[0] == N * K // 2
    # the same nibble position in both planes: 0x5 (low nibble) in plane 0, 0xA in plane 1
    lo, hi = int(p1[nz[0]]), int(p1[nz[1]])
    assert (lo, hi) in ((0x05, 0x0A), (0x50, 0xA0))


# ---------------------------------------------------------------------------
# Quality report and AWQ run-time scaling
# ---------------------------------------------------------------------------


def test_quant_error_matches_hand_computed_perturbation():
    """Symmetric 4-bit, s = 2^-6: every weight is a grid point k*s plus a known
    offset e (|e| < s/2, exact binary fraction), one weight per group is 7s so
    the scale is exactly s; the codes are k and the errors exactly e."""
    s = Fraction(1, 64)
    rng = np.random.default_rng(21)
    N, K, group = 8, 128, 32
    k = rng.integers(-6, 7, size=(N, K))
    e_num = rng.integers(-7, 8, size=(N, K))          # e = e_num * s / 16, |e| <= 7s/16 < s/2
    k[:, ::group] = 7
    e_num[:, ::group] = 0
    w_frac = [[k[n, j] * s + e_num[n, j] * s / 16 for j in range(K)] for n in range(N)]
    w = np.array([[float(v) for v in row] for row in w_frac], dtype=np.float32)
    codes, s_bits, zeros = ref.quantize_groupwise(w, group, "sym4")
    assert np.all(ref.f16_bits_to_f64(s_bits) == float(s))
    assert np.array_equal(codes.astype(np.int64) - 8, k)
    mse, snr, cos, mx = ref.quant_error(w, codes, s_bits, zeros, group)
    d2 = sum((e_num[n, j] * s / 16) ** 2 for n in range(N) for j in range(K))
    w2 = sum(v * v for row in w_frac for v in row)
    h2 = sum((k[n, j] * s) ** 2 for n in range(N) for j in range(K))
    wh = sum(w_frac[n][j] * k[n, j] * s for n in range(N) for j in range(K))
    assert mse == float(d2 / (N * K))
    assert mx == float(np.abs(e_num).max() * s / 16)
    assert abs(snr - 10 * np.log10(float(w2 / d2))) < 1e-12
    assert abs(cos - float(wh) / np.sqrt(float(w2 * h2))) < 1e-15


def test_quant_error_special_cases():
    rng = np.random.default_rng(22)
    q = rng.integers(0, 16, size=(16, 64))
    q[:, 0], q[:, 1] = 0, 15
    W = ((q - 5) * 2.0 ** -8).astype(np.float32)
    codes, s_bits, zeros = ref.quantize_groupwise(W, 64)
    mse, snr, cos, mx = ref.quant_error(W, codes, s_bits, zeros, 64)     # lattice weights: exact
    assert (mse, snr, mx) == (0.0, np.inf, 0.0) and abs(cos - 1.0) < 1e-15
    z = np.zeros((8, 32), dtype=np.float32)
    assert ref.quant_error(z, *ref.quantize_groupwise(z, 32), 32) == (0.0, np.inf, 1.0, 0.0)
    # scaling the weights by 2^e scales the error by 2^e exactly (MSE by 4^e); SNR, cosine unchanged
    w = (rng.standard_normal((16, 256)) * 0.05).astype(np.float32)
    a = ref.quant_error(w, *ref.quantize_groupwise(w, 128), 128)
    b = ref.quant_error(w * np.float32(8), *ref.quantize_groupwise(w * np.float32(8), 128), 128)
    assert b[0] == a[0] * 64 and b[3] == a[3] * 8
    assert abs(b[1] - a[1]) < 1e-9 and abs(b[2] - a[2]) < 1e-15


def test_awq_activation_rounding_matches_library_conversions():
    rng = np.random.default_rng(23)
    M, K = 4, 256
    m = (rng.uniform(0.05, 4.0, size=K)).astype(np.float32)
    for dtype in ("f16", "bf16"):
        x32 = rng.standard_normal((M, K)).astype(np.float32) * 3
        xb = ref.f32_to_f16_bits(x32) if dtype == "f16" else ref.f32_to_bf16_bits(x32)
        got = ref.awq_scale_activations(xb, dtype, m)
        x = ref.act_bits_to_f64(xb, dtype).astype(np.float32)
        prod = x * m[None, :]
        if dtype == "f16":
            want = prod.astype(np.float16).view(np.uint16)
        else:
            want = torch.from_numpy(prod).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(got, want), dtype
        assert np.array_equal(ref.awq_scale_activations(xb, dtype, np.ones(K, np.float32)), xb)


def test_awq_fold_is_exact_for_power_of_two_factors():
    """Weights scaled up by a_k = 2^e_k and activations by 1/a_k: the product of
    the quantised folded weights with the scaled activations equals x W^T of the
    unfolded lattice weights exactly."""
    rng = np.random.default_rng(24)
    N, K, group = 16, 128, 32
    q = rng.integers(0, 16, size=(N, K))
    q[:, ::group] = 0
    q[:, 1::group] = 15
    z = rng.integers(0, 16, size=(N, K // group))
    s = 2.0 ** rng.integers(-12, -6, size=(N, K // group))
    Wf = ((q - np.repeat(z, group, 1)) * np.repeat(s, group, 1)).astype(np.float32)   # folded, on the lattice
    e = rng.integers(-3, 4, size=K)
    a = np.ldexp(1.0, e).astype(np.float32)
    W = (Wf / a[None, :]).astype(np.float32)                     # the model's weights
    assert np.array_equal(ref.awq_fold_weights(W, a), Wf)
    codes, s_bits, zeros = ref.quantize_groupwise(Wf, group)
    xb = ref.f32_to_f16_bits((rng.standard_normal((3, K)) * 2).astype(np.float32))
    xs = ref.awq_scale_activations(xb, "f16", (1.0 / a).astype(np.float32))
    y, _ = ref.linear_ref_rows(xs, "f16", codes, s_bits, zeros, group)
    y_direct = ref.f16_bits_to_f64(xb) @ W.astype(np.float64).T
    assert np.allclose(y, y_direct, rtol=1e-13, atol=1e-300)


# ---------------------------------------------------------------------------
# K-quant-style super-blocks (kq4)
# ---------------------------------------------------------------------------


def test_kquant_lattice_is_reproduced_exactly():
    """Sub-blocks built as S_j q - M_j with S_j = d sc_j, M_j = dmin mq_j (d, dmin
    powers of two, one sc and one mq of 63 per super-block, q spanning 0..15)
    come back with the same codes, d, dmin, sc, mq and w_hat = w."""
    rng = np.random.default_rng(31)
    N, U = 8, 3
    K = 256 * U
    d = np.ldexp(1.0, rng.integers(-14, -8, size=(U, N)))
    dmin = d * np.ldexp(1.0, rng.integers(-3, 4, size=(U, N)))      # dmin <= 8 d
    sc = rng.integers(1, 64, size=(U, 8, N))
    sc[:, 0, :] = 63
    # M_j <= 15 S_j keeps hi = 15 S_j - M_j >= 0 (the range reading); sub-block 0
    # has sc = mq = 63 so that d and dmin are the super-block's largest / 63
    cap = np.floor(15 * sc * (d / dmin)[:, None, :]).astype(np.int64)
    mq = np.minimum(rng.integers(0, 64, size=(U, 8, N)), cap)
    mq[:, 0, :] = 63
    S = d[:, None, :] * sc
    M = dmin[:, None, :] * mq
    q = rng.integers(0, 16, size=(N, U, 8, 32))
    q[..., 0], q[..., 1] = 0, 15
    W = q * S.transpose(2, 0, 1)[..., None] - M.transpose(2, 0, 1)[..., None]
    W = W.reshape(N, K).astype(np.float32)
    assert np.array_equal(W.astype(np.float64).reshape(N, U, 8, 32),
                          q * S.transpose(2, 0, 1)[..., None] - M.transpose(2, 0, 1)[..., None])
    codes, d_bits, m_bits, sc_o, mq_o = ref.quantize_kquant(W)
    assert np.array_equal(ref.f16_bits_to_f64(d_bits), d)
    assert np.array_equal(ref.f16_bits_to_f64(m_bits), dmin)
    assert np.array_equal(sc_o, sc) and np.array_equal(mq_o, mq)
    assert np.array_equal(codes.reshape(N, U, 8, 32), q)
    assert np.array_equal(ref.dequantize_kquant(codes, d_bits, m_bits, sc_o, mq_o), W.astype(np.float64))


def test_kquant_codes_are_nearest_given_the_sub_block_parameters():
    rng = np.random.default_rng(32)
    w = (rng.standard_t(5, size=(12, 512)) * 0.02).astype(np.float32)
    w[3] = np.abs(w[3])
    w[4, :256] = 0.0
    codes, d_bits, m_bits, sc, mq = ref.quantize_kquant(w)
    S, M = ref.kquant_sub_params(d_bits, m_bits, sc, mq)
    N, K = w.shape
    grid = np.arange(16)[None, None, None, :] * S[:, :, None, None] - M[:, :, None, None]
    w64 = w.astype(np.float64).reshape(N, K // 32, 32)
    dist = np.abs(w64[..., None] - grid)
    got = np.take_along_axis(dist, codes.reshape(N, K // 32, 32, 1).astype(np.int64), axis=-1)[..., 0]
    assert np.all(got <= dist.min(-1) + 2.0 ** -20 * (np.abs(w64) + M[:, :, None]) + 1e-30)
    # the all-zero super-block: smallest scales, zero codes, exact zeros
    assert d_bits[0, 4] == 1 and m_bits[0, 4] == 1
    assert np.all(codes[4, :256] == 0) and np.all(sc[0, :, 4] == 0) and np.all(mq[0, :, 4] == 0)
    w_hat = ref.dequantize_kquant(codes, d_bits, m_bits, sc, mq)
    assert np.all(w_hat[4, :256] == 0.0)
    # one-signed positive row: no minimum
    assert np.all(mq[:, :, 3] == 0)


def test_kquant_record_layout_by_hand():
    d_bits = np.array([[0x1234]], dtype=np.uint16)
    m_bits = np.array([[0xABCD]], dtype=np.uint16)
    sc = np.array([[[1], [2], [3], [4], [5], [6], [7], [63]]], dtype=np.uint8)
    mq = np.array([[[63], [0], [0], [0], [0], [0], [0], [1]]], dtype=np.uint8)
    rec = ref.pack_kquant_records(d_bits, m_bits, sc, mq)
    scf = sum(v << (6 * j) for j, v in enumerate([1, 2, 3, 4, 5, 6, 7, 63]))
    mqf = 63 | (1 << 42)
    assert rec.shape == (1, 1, 4)
    assert rec[0, 0].tolist() == [0xABCD1234, scf & 0xFFFFFFFF, (scf >> 32) | ((mqf & 0xFFFF) << 16), mqf >> 16]
    assert rec[0, 0, 2] == 0x003FFC00 | (scf >> 32)   # mq_0 = 63 -> bits 16..21 of word 2


def test_kquant_byte_accounting():
    assert ref.format_bits_per_weight(256, "kq4") == 4.5
    q, s, z = ref.packed_bytes(5120, 13824, 256, "kq4")
    assert (q, s, z) == (5120 * 13824 // 2, 16 * 54 * 5120, 0)
    assert (q + s + z) * 8 == 5120 * 13824 * 4.5
    with pytest.raises(ValueError):
        ref.quantize_kquant(np.zeros((8, 128), np.float32))
