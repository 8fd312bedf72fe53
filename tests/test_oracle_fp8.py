"""Pins for the oracle's FP8 (e4m3) dispatch support.

- e4m3 rounding against torch's float8_e4m3fn conversion (a library
  routine) on every bf16 value and on random floats up to 464, including the
  exact midpoints between neighbouring codes; decoding of all 256 codes;
- quantisation against a numpy/torch restatement per block (amax with numpy,
  the fp32 product, torch's e4m3 rounding), and the round-trip error bound of
  a 3-bit mantissa;
- FP8 dispatch against numpy fancy indexing, for token-major and for
  TMA-aligned column-major scale layouts.
"""
import numpy as np
import pytest
import torch

import ep_inputs
import oracle


def torch_e4m3(v):
    return torch.from_numpy(np.ascontiguousarray(v, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_decode_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.e4m3_to_float(codes)
    theirs = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()
    np.testing.assert_array_equal(np.isnan(ours), np.isnan(theirs))
    ok = ~np.isnan(theirs)
    np.testing.assert_array_equal(ours[ok], theirs[ok])
    np.testing.assert_array_equal(np.signbit(ours[ok]), np.signbit(theirs[ok]))


def test_e4m3_rounding_matches_torch():
    rng = np.random.default_rng(3)
    bf = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    vals = torch.from_numpy(bf.view(np.int16)).view(torch.bfloat16).float().numpy()
    vals = vals[np.isfinite(vals) & (np.abs(vals) <= 464)]
    mags = oracle.e4m3_to_float(np.arange(0x7F, dtype=np.uint8)).astype(np.float64)
    mids = ((mags[1:] + mags[:-1]) / 2).astype(np.float32)      # exact in fp32
    rand = (rng.random(200000) * 464).astype(np.float32) * rng.choice([-1, 1], 200000).astype(np.float32)
    tiny = (rng.random(50000) * 0.02).astype(np.float32)
    v = np.concatenate([vals, mids, -mids, rand, tiny])
    np.testing.assert_array_equal(oracle.float_to_e4m3(v), torch_e4m3(v))


def test_e4m3_saturates():
    got = oracle.float_to_e4m3(np.array([465.0, 1e6, -1e30, 448.0], np.float32))
    np.testing.assert_array_equal(got, [0x7E, 0x7E, 0xFE, 0x7E])


def _restated_quantize(x_u16):
    x = torch.from_numpy(x_u16.view(np.int16)).view(torch.bfloat16).float().numpy()
    T, H = x.shape
    xb = x.reshape(T, H // 128, 128)
    amax = np.abs(xb).max(axis=2)
    inv = np.where(amax > 0, np.float32(448.0) / np.where(amax > 0, amax, 1), 0).astype(np.float32)
    v = (xb * inv[:, :, None]).astype(np.float32)
    return torch_e4m3(v.reshape(T, H)), (amax / np.float32(448.0)).astype(np.float32), x


@pytest.mark.parametrize("name", ["tiny", "decode128"])
def test_quantize_matches_restatement(name):
    inp = ep_inputs.make_inputs(name)
    q, sf = oracle.quantize_fp8(inp.x)
    q2, sf2, x = _restated_quantize(inp.x)
    np.testing.assert_array_equal(q, q2)
    np.testing.assert_array_equal(sf, sf2)
    # round trip: 3 mantissa bits -> relative error <= 2^-4, plus half the
    # subnormal step (2^-10 in scaled units)
    deq = oracle.e4m3_to_float(q).reshape(x.shape[0], -1, 128) * sf[:, :, None]
    err = np.abs(deq.reshape(x.shape) - x)
    bound = np.abs(x) * 2.0 ** -4 + np.repeat(sf, 128, axis=1) * 2.0 ** -10 * 1.0001
    assert np.all(err <= bound)


def test_quantize_zero_block_and_extremes():
    x = np.zeros((2, 256), np.uint16)
    x[1, 128] = 0x4300   # 128.0
    x[1, 129] = 0xC300   # -128.0
    x[1, 130] = 0x3F80   # 1.0
    q, sf = oracle.quantize_fp8(x)
    assert (q[0] == 0).all() and (sf[0] == 0).all() and sf[1, 0] == 0
    assert q[1, 128] == 0x7E and q[1, 129] == 0xFE and sf[1, 1] == np.float32(128.0) / np.float32(448.0)
    assert oracle.e4m3_to_float(q[1, 130:131])[0] == 3.5     # 1.0 * 448/128


@pytest.mark.parametrize("column_major", [False, True])
def test_dispatch_fp8_moves_codes_and_scales(column_major):
    inp = ep_inputs.make_inputs("tiny")
    wl = inp.wl
    S = oracle.default_rank_stride(wl.T, wl.K, wl.E, wl.R)
    lay = oracle.layout(inp.topk_idx, wl.E, wl.R, S)
    q, sf = oracle.quantize_fp8(inp.x)
    rows = wl.R * S
    rq, rsf, (ts, hs), src, rw = oracle.dispatch_fp8(q, sf, lay.token_slot, rows, inp.topk_weights,
                                                   column_major_sf=column_major)
    t_of = np.repeat(np.arange(wl.T), wl.K)
    s = lay.token_slot.ravel()
    np.testing.assert_array_equal(rq[s], q[t_of])
    nb = wl.H // 128
    for b in range(nb):
        np.testing.assert_array_equal(rsf[s * ts + b * hs], sf[t_of, b])
    np.testing.assert_array_equal(src[s], t_of)
    np.testing.assert_array_equal(rw[s], inp.topk_weights.ravel())
    if column_major:
        assert ts == 1 and hs % 4 == 0 and hs >= rows
