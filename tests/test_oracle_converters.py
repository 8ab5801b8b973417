"""Pins of the oracle's number-format converters against library routines.

Round-to-nearest into a narrow format is a monotone step function whose only
decisions sit at the midpoints between consecutive representable values.  Each
converter is therefore checked, against a library cast, at every representable
value of the target format, at every midpoint (including the overflow
midpoint above the largest finite value), and at the fp32 neighbours of both;
then on 4M uniformly random fp32 bit patterns.  Library references: numpy's
float16 cast, torch's bfloat16 and float8_e4m3fn casts.  E2M1 has no library
cast here; its reference is a brute-force nearest-grid-point search.
NaN inputs are outside the method's domain and skipped.  Decoders are checked
on every code.
"""
import numpy as np
import pytest
import torch

import oracle

RNG = np.random.default_rng(20240611)
RANDOM_BITS = RNG.integers(0, 1 << 32, size=1 << 22, dtype=np.uint64).astype(np.uint32)


def _boundary_points(pos_values):
    """fp32 test points around every rounding decision of a format whose
    non-negative finite values (ascending, including the step above the max
    used for the overflow midpoint) are given."""
    v = np.asarray(pos_values, np.float64)
    mids = (v[:-1] + v[1:]) / 2.0
    base = np.concatenate([v[:-1], mids]).astype(np.float32)
    pts = [base, np.nextafter(base, np.float32(np.inf)), np.nextafter(base, np.float32(-np.inf))]
    p = np.concatenate(pts)
    p = p[p >= 0]
    p = np.concatenate([p, -p, np.array([np.inf, -np.inf, 3e38, -3e38], np.float32)])
    return np.concatenate([p, RANDOM_BITS.view(np.float32)])


def _finite_values(decode_all, step_above):
    v = decode_all.astype(np.float64)
    v = np.unique(v[np.isfinite(v) & (v >= 0)])
    return np.append(v, v[-1] + step_above)


F16_POS = _finite_values(np.arange(1 << 16, dtype=np.uint16).view(np.float16), 32.0)
BF16_POS = _finite_values(torch.from_numpy(np.arange(1 << 16, dtype=np.uint16).view(np.int16))
                          .view(torch.bfloat16).double().numpy(), 2.0 ** 120)
E4M3_POS = _finite_values(torch.from_numpy(np.arange(256, dtype=np.uint8))
                          .view(torch.float8_e4m3fn).double().numpy(), 32.0)
E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def test_f16_against_numpy():
    x = _boundary_points(F16_POS)
    x = x[~np.isnan(x)]
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16).copy()
    ref[ref == 0x7C00] = 0x7BFF  # the library overflows to inf; scales saturate at 65504
    ref[ref == 0xFC00] = 0xFBFF
    got = oracle.f32_to_f16_sat(x)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, (x[bad[:5]], got[bad[:5]], ref[bad[:5]])


def test_bf16_against_torch():
    x = _boundary_points(BF16_POS)
    x = x[~np.isnan(x)]
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.f32_to_bf16(x)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, (x[bad[:5]], got[bad[:5]], ref[bad[:5]])


def test_e4m3_against_torch_below_saturation():
    x = _boundary_points(E4M3_POS)
    x = x[~np.isnan(x) & (np.abs(x) < 464.0)]  # |x| >= 464 saturates, tested below
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = oracle.f32_to_e4m3_sat(x)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, (x[bad[:5]], got[bad[:5]], ref[bad[:5]])


def test_e4m3_saturation():
    x = np.array([455.0, 463.99, 464.0, 479.0, 480.0, 1e6, 3e38, np.inf], np.float32)
    assert np.all(oracle.f32_to_e4m3_sat(x) == 0x7E)
    assert np.all(oracle.f32_to_e4m3_sat(-x) == 0xFE)


def _e2m1_brute(x):
    """Nearest E2M1 magnitude, ties to the even code; sign bit from the input."""
    a = np.minimum(np.abs(x.astype(np.float64)), 1e3)
    d = np.abs(a[:, None] - E2M1_GRID[None, :])
    cand = d == d.min(axis=1, keepdims=True)
    even = cand & (np.arange(8) % 2 == 0)[None, :]
    idx = np.where(even.any(axis=1), np.argmax(even, axis=1), np.argmax(cand, axis=1))
    sign = np.signbit(x).astype(np.uint8) << 3
    return idx.astype(np.uint8) | sign


def test_e2m1_against_brute_force():
    x = _boundary_points(np.append(E2M1_GRID, 8.0))
    x = x[~np.isnan(x)]
    got = oracle.f32_to_e2m1_sat(x)
    ref = _e2m1_brute(x)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, (x[bad[:5]], got[bad[:5]], ref[bad[:5]])


def test_e2m1_ties_table():
    # midpoints go to the even code: .25->0, .75->1.0, 1.25->1.0, 1.75->2.0,
    # 2.5->2.0, 3.5->4.0, 5->4.0; above 6 saturates to 6; -tiny -> negative zero
    x = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0, 100.0, -0.1], np.float32)
    assert list(oracle.f32_to_e2m1_sat(x)) == [0, 2, 2, 4, 4, 6, 6, 7, 7, 8]


def test_decoders_every_code():
    h = np.arange(1 << 16, dtype=np.uint16)
    ref16 = h.view(np.float16).astype(np.float32)
    got16 = oracle.f16_to_f32(h)
    assert np.array_equal(np.isnan(ref16), np.isnan(got16))
    m = ~np.isnan(ref16)
    assert np.array_equal(ref16[m].view(np.uint32), got16[m].view(np.uint32))
    refb = torch.from_numpy(h.view(np.int16)).view(torch.bfloat16).float().numpy()
    gotb = oracle.bf16_to_f32(h)
    m = ~np.isnan(refb)
    assert np.array_equal(np.isnan(refb), np.isnan(gotb))
    assert np.array_equal(refb[m].view(np.uint32), gotb[m].view(np.uint32))
    b = np.arange(256, dtype=np.uint8)
    ref8 = torch.from_numpy(b).view(torch.float8_e4m3fn).float().numpy()
    got8 = oracle.e4m3_to_f32(b)
    m = ~np.isnan(ref8)
    assert np.array_equal(np.isnan(ref8), np.isnan(got8))
    assert np.array_equal(ref8[m].view(np.uint32), got8[m].view(np.uint32))
    c = np.arange(16, dtype=np.uint8)
    want = np.concatenate([E2M1_GRID, -E2M1_GRID]).astype(np.float32)
    assert np.array_equal(oracle.e2m1_to_f32(c).view(np.uint32), want.view(np.uint32))


@pytest.mark.parametrize("enc,dec", [(oracle.f32_to_f16_sat, oracle.f16_to_f32),
                                     (oracle.f32_to_bf16, oracle.bf16_to_f32)])
def test_roundtrip_of_representable_values(enc, dec):
    h = np.arange(1 << 16, dtype=np.uint16)
    v = dec(h)
    keep = np.isfinite(v)
    assert np.array_equal(enc(v[keep]), h[keep])
