"""Pins of the oracle's FP8 E4M3 decoding and FP8-weight expert FFN (CPU only).

FP8 expert weights are the form in which the ExpertPlex page ("Experimental
results", models table) serves GLM-5.1-FP8; the oracle reads them as OCP E4M3
codes with one fp32 scale per weight row.  The decoder is checked against
torch's float8_e4m3fn for all 256 codes and at the format's landmarks; the
FFN is checked against the plain fp32 FFN on weights that are exact in both.
"""
import numpy as np
import torch

from oracle import moe_oracle as O


def test_all_codes_match_torch_float8_e4m3fn():
    codes = np.arange(256, dtype=np.uint8)
    ours = O.fp8_e4m3_to_f64(codes)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


def test_landmark_codes():
    v = O.fp8_e4m3_to_f64(np.array([0x38, 0x7E, 0x01, 0x08, 0x07, 0x80, 0xB8, 0x3C], dtype=np.uint8))
    assert v[0] == 1.0 and v[1] == 448.0 and v[2] == 2.0 ** -9 and v[3] == 2.0 ** -6
    assert v[4] == 7 * 2.0 ** -9 and v[5] == 0.0 and np.signbit(v[5]) and v[6] == -1.0 and v[7] == 1.5
    assert np.isnan(O.fp8_e4m3_to_f64(np.array([0x7F, 0xFF], dtype=np.uint8))).all()


def test_fp8_ffn_equals_fp32_ffn_on_exact_weights():
    rng = np.random.default_rng(0)
    E, S, d, I, N = 3, 1, 16, 24, 20
    codes = lambda *shape: rng.integers(0, 256, size=shape).astype(np.uint8) & np.uint8(0x77)  # finite, |v| < 240
    qg, qu, qd = codes(E + S, I, d), codes(E + S, I, d), codes(E + S, d, I)
    # power-of-two scales: every dequantised weight is exact in float32
    sg = np.exp2(rng.integers(-8, -2, size=(E + S, I))).astype(np.float32)
    su = np.exp2(rng.integers(-8, -2, size=(E + S, I))).astype(np.float32)
    sd = np.exp2(rng.integers(-8, -2, size=(E + S, d))).astype(np.float32)
    x = rng.normal(size=(N, d)).astype(np.float32)
    offs = np.array([0, 5, 5, 12, 20], dtype=np.int32)            # 3 routed groups + 1 shared
    got = O.grouped_ffn_fp8w(x, offs, E, S, 1, qg, sg, qu, su, qd, sd, dtype="f32")
    wg = (O.fp8_e4m3_to_f64(qg) * sg[..., None]).astype(np.float32)
    wu = (O.fp8_e4m3_to_f64(qu) * su[..., None]).astype(np.float32)
    wd = (O.fp8_e4m3_to_f64(qd) * sd[..., None]).astype(np.float32)
    ref = O.grouped_ffn(x, offs, E, S, 1, wg, wu, wd, "f32")
    assert np.array_equal(got, ref)


def test_fp8_ffn_scale_is_per_output_row():
    # doubling one gate row's scale doubles exactly that SwiGLU column's gate input
    rng = np.random.default_rng(1)
    d, I = 8, 4
    q = lambda *shape: (rng.integers(0, 256, size=shape).astype(np.uint8) & np.uint8(0x57))
    qg, qu, qd = q(1, I, d), q(1, I, d), q(1, d, I)
    ones = lambda n: np.ones((1, n), dtype=np.float32)
    x = rng.normal(size=(3, d)).astype(np.float32)
    offs = np.array([0, 3], dtype=np.int32)
    base = O.grouped_ffn_fp8w(x, offs, 1, 0, 1, qg, ones(I), qu, ones(I), qd, ones(d), dtype="f32")
    sg = ones(I)
    sg[0, 2] = 2.0
    scaled = O.grouped_ffn_fp8w(x, offs, 1, 0, 1, qg, sg, qu, ones(I), qd, ones(d), dtype="f32")
    wg = O.fp8_e4m3_to_f64(qg[0]); wu = O.fp8_e4m3_to_f64(qu[0]); wd = O.fp8_e4m3_to_f64(qd[0])
    xs = x.astype(np.float64)
    g, u = xs @ wg.T, xs @ wu.T
    g2 = g.copy(); g2[:, 2] *= 2
    delta = (O.silu_product(g2, u) - O.silu_product(g, u)) @ wd.T
    assert np.allclose(scaled - base, delta, rtol=1e-12, atol=1e-12)
