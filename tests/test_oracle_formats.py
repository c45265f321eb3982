"""Pins of the oracle's format decoders and of the generator's encoders."""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def test_e4m3_spec_values():
    g = _gold("format_values.json")
    for code, val in g["e4m3"].items():
        got = oracle.E4M3_TABLE[int(code, 16)]
        if val == "nan":
            assert math.isnan(got)
        else:
            assert got == val and math.copysign(1, got) == math.copysign(1, val), code
    finite = oracle.E4M3_TABLE[np.isfinite(oracle.E4M3_TABLE)]
    assert finite.max() == g["e4m3_max_normal"]
    assert np.min(np.abs(finite[finite != 0])) == g["e4m3_min_subnormal"]
    assert np.isnan(oracle.E4M3_TABLE).sum() == 2


def test_e4m3_matches_torch_float8():
    """Library cross-check: torch's float8_e4m3fn decode of all 256 codes."""
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    mine = oracle.E4M3_TABLE
    both_nan = np.isnan(ref) & np.isnan(mine)
    assert np.array_equal(ref[~both_nan], mine[~both_nan])
    assert both_nan.sum() == 2


def test_e2m1_spec_values():
    g = _gold("format_values.json")
    mags = oracle.E2M1_TABLE[:8]
    assert list(mags) == g["e2m1_magnitudes"]
    assert list(oracle.E2M1_TABLE[8:]) == [-m for m in g["e2m1_magnitudes"]]
    assert oracle.E2M1_TABLE.max() == g["e2m1_max"]


def test_bf16_decode_matches_torch():
    bits = torch.randint(-32768, 32767, (4096,), dtype=torch.int16,
                         generator=torch.Generator().manual_seed(5))
    ref = bits.view(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.decode_bf16(bits.numpy())
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], got[ok])


def test_fp4_record_hand_decoded():
    """Element 2i sits in the low nibble of byte i; scale g covers elements
    32g..32g+31."""
    rec = np.zeros((1, 320), dtype=np.uint8)
    rec[0, 0] = 0x71          # element 0 = code 1 (0.5), element 1 = code 7 (6)
    rec[0, 15] = 0xA3         # element 30 = code 3 (1.5), element 31 = code 0xA (-1)
    rec[0, 16] = 0x0E         # element 32 = code 0xE (-4)
    scales = np.array([2.0] + [0.25] * 15, dtype="<f4")
    rec[0, 256:] = scales.view(np.uint8)
    v = oracle.decode_fp4_records(rec)[0]
    assert v[0] == 1.0 and v[1] == 12.0
    assert v[30] == 3.0 and v[31] == -2.0
    assert v[32] == -1.0 and v[33] == 0.0
    assert np.count_nonzero(v) == 5


def test_swa_record_hand_decoded():
    rec = np.zeros((1, 528), dtype=np.uint8)
    rec[0, 0] = 0x38          # 1.0
    rec[0, 127] = 0xBC        # -1.5
    rec[0, 128] = 0x40        # 2.0
    rec[0, 511] = 0x7E        # 448
    rec[0, 512:] = np.array([3.0, 0.5, 1.0, 0.125], dtype="<f4").view(np.uint8)
    v = oracle.decode_swa_records(rec)[0]
    assert v[0] == 3.0 and v[127] == -4.5 and v[128] == 1.0 and v[511] == 56.0
    assert np.count_nonzero(v) == 4


def test_fp4s16_rows_hand_decoded():
    """The pages' FP4 format: element 2i in the low nibble of byte i, E4M3
    scale byte g covering elements 16g..16g+15."""
    codes = np.zeros((1, 64), dtype=np.uint8)
    scales = np.zeros((1, 8), dtype=np.uint8)
    codes[0, 0] = 0x71        # element 0 = code 1 (0.5), element 1 = code 7 (6)
    codes[0, 7] = 0xA3        # element 14 = code 3 (1.5), element 15 = code 0xA (-1)
    codes[0, 8] = 0x0E        # element 16 = code 0xE (-4)
    codes[0, 63] = 0x50       # element 127 = code 5 (3)
    scales[0] = [0x40, 0x30, 0, 0, 0, 0, 0, 0x01]   # 2.0, 0.5, ..., 2^-9
    v = oracle.decode_fp4s16_rows(codes, scales)[0]
    assert v.shape == (128,)
    assert v[0] == 1.0 and v[1] == 12.0 and v[14] == 3.0 and v[15] == -2.0
    assert v[16] == -2.0 and v[127] == 3.0 * 2.0 ** -9
    assert np.count_nonzero(v) == 6


def test_fp4s16_values_are_exact_in_f16():
    """Every finite E2M1 code times every finite E4M3 scale is an f16 value:
    the kernels widen these rows to f16 without rounding."""
    e2m1 = oracle.E2M1_TABLE
    e4m3 = oracle.E4M3_TABLE[np.isfinite(oracle.E4M3_TABLE)]
    prod = np.outer(e2m1, e4m3).ravel()
    assert np.array_equal(prod.astype(np.float16).astype(np.float64), prod)


def _nearest_grid_ok(x, decoded, grid):
    """decoded must be a nearest grid point of x (ties: either neighbour)."""
    dist = np.abs(x[..., None] - grid)
    best = dist.min(axis=-1)
    return np.all(np.abs(x - decoded) <= best + 1e-12 * np.maximum(1, np.abs(x)))


def test_generator_e4m3_rows_round_to_nearest():
    x = torch.randn(64, 128, generator=torch.Generator().manual_seed(1)) * 3
    codes, scale = synth.encode_e4m3_rows(x)
    assert scale.shape == (64, 1)
    scale = scale[:, 0]
    xs = x.numpy().astype(np.float64)
    amax = np.abs(x.numpy()).max(axis=1)
    assert np.array_equal(scale.numpy(), amax / np.float32(448.0))
    dec = oracle.decode_e4m3_rows(codes.numpy(), np.ones(64))
    grid = oracle.E4M3_TABLE[np.isfinite(oracle.E4M3_TABLE)]
    y = (torch.from_numpy(xs).float() / scale[:, None]).double().numpy()
    assert _nearest_grid_ok(y, dec, grid)


def test_generator_fp4_records_round_to_nearest():
    x = torch.randn(32, 512, generator=torch.Generator().manual_seed(2))
    rec = synth.encode_fp4_records(x)
    assert rec.shape == (32, synth.FP4_RECORD_BYTES) == (32, 320)
    scales = rec[:, 256:].contiguous().view(torch.float32).numpy()
    g = x.reshape(32, 16, 32).abs().amax(dim=2).numpy()
    assert np.array_equal(scales, (g / np.float32(6.0)).astype(np.float32))
    dec = oracle.decode_fp4_records(rec.numpy())
    y = (x.reshape(32, 16, 32) / torch.from_numpy(scales)[:, :, None]).reshape(32, 512)
    grid = oracle.E2M1_TABLE
    dec_unscaled = dec / np.repeat(scales.astype(np.float64), 32, axis=1)
    assert _nearest_grid_ok(y.double().numpy(), dec_unscaled, grid)


def test_generator_fp4_ties_to_even():
    """Midpoints of the E2M1 grid round to the even-mantissa neighbour."""
    mids = torch.tensor([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    expect = [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0]
    row = torch.zeros(1, 512)
    row[0, :7] = mids
    row[0, 31] = 6.0          # group amax 6 -> scale exactly 1
    dec = oracle.decode_fp4_records(synth.encode_fp4_records(row).numpy())[0]
    assert list(dec[:7]) == expect


def test_generator_swa_records():
    x = torch.randn(8, 512, generator=torch.Generator().manual_seed(3))
    rec = synth.encode_swa_records(x)
    assert rec.shape == (8, synth.SWA_RECORD_BYTES) == (8, 528)
    dec = oracle.decode_swa_records(rec.numpy())
    rel = np.abs(dec - x.numpy()) / np.repeat(np.abs(x.numpy()).reshape(8, 4, 128).max(2), 128, 1)
    assert rel.max() <= 2.0 ** -4 * 448 / 448 + 1e-7   # half an E4M3 ulp at the top binade


def test_generator_is_deterministic():
    a = synth.mini_workload(7, [100, 37], q_per_seq=2, quantized=True)
    b = synth.mini_workload(7, [100, 37], q_per_seq=2, quantized=True)
    for x, y in [(a.k_idx, b.k_idx), (a.main_kv, b.main_kv), (a.layers[0].q, b.layers[0].q),
                 (a.layers[0].swa, b.layers[0].swa)]:
        assert torch.equal(x, y)
    c = synth.mini_workload(8, [100, 37], q_per_seq=2, quantized=True)
    assert not torch.equal(a.k_idx, c.k_idx)


def test_generator_fp4s16_rows():
    """Scale = amax/16-group / 6 rounded to E4M3; each element is a nearest
    E2M1 point of value / decoded scale (saturating at 6)."""
    x = torch.randn(48, 128, generator=torch.Generator().manual_seed(5))
    codes, scales = synth.encode_fp4s16_rows(x)
    assert codes.shape == (48, 64) and scales.shape == (48, 8)
    amax = x.reshape(48, 8, 16).abs().amax(dim=2)
    want = (amax / 6.0).to(torch.float8_e4m3fn).view(torch.uint8)
    assert torch.equal(scales, want)
    sdec = oracle.E4M3_TABLE[scales.numpy()]
    dec = oracle.decode_fp4s16_rows(codes.numpy(), scales.numpy())
    y = (x.double().numpy().reshape(48, 8, 16) / sdec[:, :, None]).reshape(48, 128)
    y = np.clip(y, -6.0, 6.0)
    assert _nearest_grid_ok(y, dec / np.repeat(sdec, 16, axis=1), oracle.E2M1_TABLE)


def test_fp4s16_record_hand_decoded():
    """The pages' 288-byte record: 256 code bytes, then one E4M3 scale byte per
    16 elements."""
    rec = np.zeros((1, 288), dtype=np.uint8)
    rec[0, 0] = 0x71          # elements 0, 1 = 0.5, 6
    rec[0, 255] = 0x90        # element 510 = 0, element 511 = code 9 (-0.5)
    rec[0, 256] = 0x40        # scale of elements 0..15: 2.0
    rec[0, 287] = 0x7E        # scale of elements 496..511: 448
    v = oracle.decode_fp4s16_records(rec)[0]
    assert v.shape == (512,)
    assert v[0] == 1.0 and v[1] == 12.0 and v[511] == -224.0
    assert np.count_nonzero(v) == 3


def test_generator_fp4s16_records():
    x = torch.randn(16, 512, generator=torch.Generator().manual_seed(6))
    rec = synth.encode_fp4s16_records(x)
    assert rec.shape == (16, synth.FP4S16_RECORD_BYTES) == (16, 288)
    codes, scales = synth.encode_fp4s16_rows(x)
    assert torch.equal(rec[:, :256], codes) and torch.equal(rec[:, 256:], scales)
    assert np.array_equal(oracle.decode_fp4s16_records(rec.numpy()),
                          oracle.decode_fp4s16_rows(codes.numpy(), scales.numpy()))
