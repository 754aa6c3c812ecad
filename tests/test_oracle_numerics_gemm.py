"""Pins for oracle.numerics (against torch's CPU casts, exhaustively where the
input space allows) and oracle.gemm (explicit sums, exact rational arithmetic)."""

from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import gemm, numerics


def test_bf16_rne_matches_torch_over_all_bf16_neighbourhoods():
    hi = np.arange(65536, dtype=np.uint32)
    for lo in (0, 1, 0x7FFF, 0x8000, 0x8001, 0xFFFF, 0x4000, 0xC000):
        u = (hi << 16) | lo
        f = u.view(np.float32)
        ours = numerics.f32_to_bf16_bits(f)
        ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        finite = np.isfinite(f)
        assert np.array_equal(ours[finite], ref[finite])
        nan = np.isnan(f)
        assert np.isnan(numerics.bf16_bits_to_f64(ours[nan])).all()


def test_bf16_to_f64_is_exact():
    bits = np.arange(65536, dtype=np.uint16)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
    ours = numerics.bf16_bits_to_f64(bits)
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok]) and np.isnan(ours[~ok]).all()


def test_e4m3_decode_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).double().numpy()
    ours = numerics.e4m3_to_f64(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert ours[0x7E] == 448.0 and ours[0x01] == 2.0 ** -9


def test_e4m3_encode_matches_torch_in_range():
    rng = np.random.default_rng(0)
    vals = numerics.e4m3_to_f64(np.arange(0, 0x7F))
    mids = (vals[:-1] + vals[1:]) / 2
    x = np.concatenate([vals, mids, -mids, mids * (1 + 1e-7), mids * (1 - 1e-7),
                        rng.uniform(-464, 464, 20000), rng.normal(0, 1, 20000),
                        np.array([0.0, -0.0, 464.0, -464.0, 1e-12])])
    x32 = x.astype(np.float32)
    ours = numerics.f64_to_e4m3(x32.astype(np.float64))
    ref = torch.from_numpy(x32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_e4m3_encode_saturates_and_nan():
    out = numerics.f64_to_e4m3(np.array([465.0, 1e9, -1e9, np.inf, -np.inf, np.nan]))
    assert list(out) == [0x7E, 0x7E, 0xFE, 0x7E, 0xFE, 0x7F]


def test_int4_dequant_matches_torch():
    rng = np.random.default_rng(1)
    q = rng.integers(0, 16, (64, 256)).astype(np.uint8)
    sc = torch.from_numpy(rng.normal(0.01, 0.002, (64, 2)).astype(np.float32)).to(torch.bfloat16)
    sbits = sc.view(torch.int16).numpy().view(np.uint16)
    ours = numerics.int4_dequant_bf16_bits(q, sbits)
    ref = ((torch.from_numpy(q.astype(np.float32)) - 8.0)
           * sc.float().repeat_interleave(128, dim=1)).to(torch.bfloat16)
    assert np.array_equal(ours, ref.view(torch.int16).numpy().view(np.uint16))


def _torch_fp8_quant(bits):
    """The same per-tensor quantisation in torch CPU float32: inv = 448 / amax
    and sx = amax / 448 as fp32 divisions (correctly rounded), the product
    x * inv in fp32, then torch's e4m3 cast (round to nearest even)."""
    x = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).float()
    amax = x.abs().max()
    inv = torch.tensor(448.0, dtype=torch.float32) / amax
    sx = amax / torch.tensor(448.0, dtype=torch.float32)
    q = (x * inv).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return q, float(sx)


def _bf16_bits(values):
    return torch.tensor(values, dtype=torch.float32).to(torch.bfloat16).view(
        torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("seed,scale", [(2, 1.0), (3, 1e-3), (4, 300.0), (5, 0.0)])
def test_fp8_activation_quant_bit_exact_against_torch_float32(seed, scale):
    rng = np.random.default_rng(seed)
    if scale:
        v = rng.normal(0, scale, (16, 512))
    else:  # magnitudes spread over 2^-30 .. 2^8, so the e4m3 subnormals are hit
        v = np.exp2(rng.uniform(-30, 8, (16, 512))) * rng.choice([-1.0, 1.0], (16, 512))
    bits = _bf16_bits(v)
    xq, sx = numerics.fp8_quantize_activations(bits)
    rq, rsx = _torch_fp8_quant(bits)
    assert np.array_equal(xq, rq)
    assert sx == rsx


def test_fp8_activation_quant_ties_round_to_even():
    # amax = 448 makes inv = 1 exactly: these bf16 values are e4m3 midpoints
    x = [448.0, 1.0625, 1.1875, -1.0625, 432.0, 2.0 ** -10, 3 * 2.0 ** -10, 0.0]
    want = [0x7E, 0x38, 0x3A, 0xB8, 0x7E, 0x00, 0x02, 0x00]
    bits = _bf16_bits(x)
    xq, sx = numerics.fp8_quantize_activations(bits)
    assert sx == 1.0 and xq.tolist() == want
    assert _torch_fp8_quant(bits)[0].tolist() == want


# (amax, x) where the exact x * inv and its fp32 rounding fall on different
# sides of an e4m3 rounding boundary: only the fp32 product gives torch's code
FP32_STEP_CASES = [(0.5234375, 2.396106719970703e-05), (0.5234375, 4.792213439941406e-05),
                   (3.171875, 2.0742416381835938e-05), (29.125, 0.0004444122314453125),
                   (0.0002269744873046875, 4.94765117764473e-10)]


@pytest.mark.parametrize("amax,x", FP32_STEP_CASES)
def test_fp8_activation_quant_rounds_the_product_to_fp32_first(amax, x):
    bits = _bf16_bits([amax, x, -x])
    xq, sx = numerics.fp8_quantize_activations(bits)
    rq, rsx = _torch_fp8_quant(bits)
    assert xq.tolist() == rq.tolist() and sx == rsx
    # the product rounded straight from its exact value would give another code
    inv = float(np.float32(448.0 / float(numerics.bf16_bits_to_f64(bits[:1])[0])))
    exact = float(numerics.bf16_bits_to_f64(bits[1:2])[0]) * inv
    assert int(numerics.f64_to_e4m3(np.array([exact]))[0]) != int(xq[1])


def test_fp8_activation_quant_properties():
    rng = np.random.default_rng(2)
    x = torch.from_numpy(rng.normal(0, 1, (8, 512)).astype(np.float32)).to(torch.bfloat16)
    bits = x.view(torch.int16).numpy().view(np.uint16)
    xq, sx = numerics.fp8_quantize_activations(bits)
    xv = x.double().numpy()
    amax = np.abs(xv).max()
    assert sx == pytest.approx(amax / 448, rel=2 ** -23)
    # the largest element maps to +-448
    i = np.unravel_index(np.abs(xv).argmax(), xv.shape)
    assert numerics.e4m3_to_f64(xq[i]) == pytest.approx(448.0 * np.sign(xv[i]))
    # dequantised values are within half an e4m3 ulp (relative 2^-4) or the subnormal step
    back = numerics.e4m3_to_f64(xq) * sx
    err = np.abs(back - xv)
    assert (err <= np.maximum(np.abs(xv) * 2.0 ** -4, sx * 2.0 ** -10) * 1.0001).all()
    z, s0 = numerics.fp8_quantize_activations(np.zeros((2, 4), np.uint16))
    assert (z == 0).all() and s0 == 1.0


# ------------------------------------------------------------------ gemm
def test_gemm_matches_explicit_sums():
    rng = np.random.default_rng(3)
    x = rng.normal(size=(5, 37))
    w = rng.normal(size=(11, 37))
    assert np.allclose(gemm.gemm_fp64(x, w), gemm.gemm_loop(x, w), rtol=1e-13, atol=1e-13)


def test_gemm_exact_against_fractions():
    rng = np.random.default_rng(4)
    xb = numerics.f32_to_bf16_bits(rng.normal(size=(3, 8)).astype(np.float32))
    wb = numerics.f32_to_bf16_bits(rng.normal(size=(4, 8)).astype(np.float32))
    x = numerics.bf16_bits_to_f64(xb)
    w = numerics.bf16_bits_to_f64(wb)
    y = gemm.gemm_fp64(x, w)
    for i in range(3):
        for j in range(4):
            exact = sum(Fraction(float(x[i, t])) * Fraction(float(w[j, t])) for t in range(8))
            assert abs(Fraction(float(y[i, j])) - exact) <= abs(exact) * Fraction(1, 2 ** 50)


def test_gemm_transpose_orientation():
    # Y = X W^T: W rows are output features
    x = np.array([[1.0, 2.0, 3.0]])
    w = np.array([[1.0, 0.0, 0.0], [0.0, 0.0, 1.0]])
    assert gemm.gemm_fp64(x, w).tolist() == [[1.0, 3.0]]


def test_weight_values_per_format():
    codes8 = np.array([[-127, -1, 0, 5]], dtype=np.int8)
    assert gemm.weight_values(gemm.FMT_INT8, codes8).tolist() == [[-127, -1, 0, 5]]
    b = np.array([[0x3F80, 0xBF80, 0x4040]], dtype=np.uint16)
    assert gemm.weight_values(gemm.FMT_BF16, b).tolist() == [[1.0, -1.0, 3.0]]
    f8 = np.array([[0x38, 0xB8, 0x7E]], dtype=np.uint8)
    assert gemm.weight_values(gemm.FMT_FP8, f8).tolist() == [[1.0, -1.0, 448.0]]
    q = np.full((1, 128), 10, dtype=np.uint8)
    s = np.array([[0x3F00]], dtype=np.uint16)  # 0.5
    assert (gemm.weight_values(gemm.FMT_INT4, q, s) == 1.0).all()


def test_reference_output_fp8_exact_case():
    # X already on the e4m3 grid with amax 448 -> sx = 1, and W scale 0.5
    x = np.array([[448.0, -1.0, 0.5, 0.0]], dtype=np.float32)
    xb = numerics.f32_to_bf16_bits(x)
    wq = numerics.f64_to_e4m3(np.array([[1.0, 2.0, 4.0, 8.0], [-1.0, 0.0, 0.0, 448.0]]))
    y = gemm.reference_output(gemm.FMT_FP8, wq, xb, w_scale=0.5)
    assert y.tolist() == [[0.5 * (448 - 2 + 2), 0.5 * (-448)]]


# ------------------------------------------------------------ rel_frobenius
def test_rel_frobenius_hand_computed():
    y = np.array([[1.0, 2.0], [3.0, 4.0]])
    ref = np.array([[1.0, 2.0], [3.0, 5.0]])
    # |y - ref|_F = 1, |ref|_F = sqrt(1 + 4 + 9 + 25)
    assert gemm.rel_frobenius(y, ref) == pytest.approx(1.0 / np.sqrt(39.0), rel=1e-15)
    assert gemm.rel_frobenius(ref, ref) == 0.0
    # a zero reference: the plain Frobenius norm of the difference
    assert gemm.rel_frobenius(np.array([[3.0, 4.0]]), np.zeros((1, 2))) == 5.0


def test_rel_frobenius_fails_a_perturbed_output():
    """Negative control of the 1e-5 parity bound: one element off by 2e-5 of
    the reference's norm, or one element never written (NaN), must fail it."""
    rng = np.random.default_rng(9)
    ref = rng.normal(size=(16, 256))
    y = ref.copy()
    y[3, 17] += 2e-5 * np.linalg.norm(ref)
    err = gemm.rel_frobenius(y, ref)
    assert err == pytest.approx(2e-5, rel=1e-6) and not err <= 1e-5
    y = ref.astype(np.float32).astype(np.float64)
    assert gemm.rel_frobenius(y, ref) <= 1e-7  # an fp32 rounding of every element passes
    y[0, 0] = np.nan
    assert not gemm.rel_frobenius(y, ref) <= 1e-5
