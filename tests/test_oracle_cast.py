"""Pins of the oracle's half <-> fp32 conversions and overflow test (CPU only).

Checked against library conversions (numpy float16, torch float16 / bfloat16),
which implement IEEE 754 round-to-nearest-even, over every half bit pattern,
over a structured sweep of fp32 patterns that hits every exponent, both
parities of the last kept bit, exact ties and their neighbours, and over all
2^32 fp32 bit patterns (the last two tests, run in chunks on all cores).
"""
import numpy as np
import pytest
import torch

import oracle

ALL16 = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)


def _bf16_to_f32_torch(bits):
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()


def _f32_to_bf16_torch(x):
    return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _sweep_f32():
    """All 2^16 top halves x 64 low patterns (bits 13..15 x tie-region patterns) + random."""
    lows = []
    for b in range(8):
        for lo in (0x0000, 0x0001, 0x0FFF, 0x1000, 0x1001, 0x1FFF, 0x0ABC, 0x1555):
            lows.append((b << 13) | lo)
    lows = np.array(sorted(set(lows)), dtype=np.uint32)
    hi = np.arange(1 << 16, dtype=np.uint32) << 16
    pats = (hi[:, None] | lows[None, :]).ravel()
    rnd = np.random.default_rng(0).integers(0, 1 << 32, size=1 << 21, dtype=np.uint64)
    return np.concatenate([pats, rnd.astype(np.uint32)]).view(np.float32)


def test_f16_to_f32_exhaustive():
    got = oracle.half_to_float(ALL16, "f16")
    ref = ALL16.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))
    assert np.array_equal(np.signbit(got), np.signbit(ref))


def test_bf16_to_f32_exhaustive():
    got = oracle.half_to_float(ALL16, "bf16")
    ref = _bf16_to_f32_torch(ALL16)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_f32_to_f16_rne_sweep():
    x = _sweep_f32()
    got = oracle.float_to_half(x, "f16")
    with np.errstate(over="ignore", invalid="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    nan = np.isnan(x)
    assert np.array_equal(got[~nan], ref[~nan])
    # NaN stays NaN (quiet) with its sign
    gn = got[nan]
    assert np.all((gn & 0x7C00) == 0x7C00) and np.all((gn & 0x03FF) != 0)
    assert np.all((gn & 0x0200) != 0)
    assert np.array_equal(gn >> 15, (x[nan].view(np.uint32) >> 31).astype(np.uint16))


def test_f32_to_bf16_rne_sweep():
    x = _sweep_f32()
    got = oracle.float_to_half(x, "bf16")
    ref = _f32_to_bf16_torch(x)
    nan = np.isnan(x)
    assert np.array_equal(got[~nan], ref[~nan])
    gn = got[nan]
    assert np.all((gn & 0x7F80) == 0x7F80) and np.all((gn & 0x0040) != 0)


def test_round_trip_of_every_half_value():
    for dt in ("f16", "bf16"):
        f = oracle.half_to_float(ALL16, dt)
        back = oracle.float_to_half(f, dt)
        finite = ~np.isnan(f)
        assert np.array_equal(back[finite], ALL16[finite])


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_nonfinite_exhaustive(dt):
    if dt == "f16":
        bad = ~np.isfinite(ALL16.view(np.float16))
    else:
        bad = ~np.isfinite(_bf16_to_f32_torch(ALL16))
    got = np.array([oracle.nonfinite(ALL16[i:i + 1], dt) for i in range(1 << 16)])
    assert np.array_equal(got, bad)
    # largest finite values, subnormals and -0 do not trip; inf and NaN do
    fin = {"f16": [0x7BFF, 0xFBFF, 0x0001, 0x8000], "bf16": [0x7F7F, 0xFF7F, 0x0001, 0x8000]}[dt]
    assert not oracle.nonfinite(np.array(fin, dtype=np.uint16), dt)
    special = {"f16": [0x7C00, 0xFC00, 0x7E00, 0x7C01], "bf16": [0x7F80, 0xFF80, 0x7FC0, 0x7F81]}
    for h in special[dt]:
        arr = np.zeros(1000, dtype=np.uint16)
        arr[999] = h
        assert oracle.nonfinite(arr, dt)


def test_nonfinite_f32_sweep():
    # every sign / exponent / top-7-fraction-bit pattern (the high half-word),
    # each with low half-words 0, 1, 0x8000 and 0xFFFF, against numpy's isfinite
    hi = np.arange(1 << 16, dtype=np.uint32) << 16
    words = (hi[:, None] | np.array([0x0000, 0x0001, 0x8000, 0xFFFF], np.uint32)[None, :]).ravel()
    bad = ~np.isfinite(words.view(np.float32))
    got = np.array([oracle.nonfinite(words[i:i + 1], "f32") for i in range(words.size)])
    assert np.array_equal(got, bad)
    # largest finite values, the smallest subnormal and -0 do not trip; inf and NaN do
    fin = np.array([0x7F7FFFFF, 0xFF7FFFFF, 0x00000001, 0x80000000], np.uint32)
    assert not oracle.nonfinite(fin, "f32")
    for w in (0x7F800000, 0xFF800000, 0x7FC00000, 0x7F800001):
        arr = np.zeros(1000, dtype=np.uint32)
        arr[999] = w
        assert oracle.nonfinite(arr, "f32")


def _all_2_32(dt, ref_fn):
    """oracle.float_to_half over all 2^32 fp32 patterns against ref_fn, in
    2^24-pattern chunks on a thread pool (ctypes and torch release the GIL).
    Non-NaN inputs must match bit for bit; NaN must give a quiet NaN of the
    same sign."""
    import os
    from concurrent.futures import ThreadPoolExecutor
    chunk = 1 << 24
    emask, quiet = (0x7C00, 0x0200) if dt == "f16" else (0x7F80, 0x0040)

    def run(c):
        u = (np.arange(chunk, dtype=np.uint64) + c * chunk).astype(np.uint32)
        x = u.view(np.float32)
        got = oracle.float_to_half(x, dt)
        ref = ref_fn(x)
        nan = np.isnan(x)
        bad = np.flatnonzero((got != ref) & ~nan)
        gn = got[nan]
        nan_ok = bool(np.all((gn & emask) == emask) and np.all((gn & quiet) != 0) and
                      np.array_equal(gn >> 15, (u[nan] >> 31).astype(np.uint16)))
        return [hex(int(u[i])) for i in bad[:4]], int(bad.size), nan_ok

    workers = max(1, min(16, os.cpu_count() or 1))
    threads = torch.get_num_threads()
    torch.set_num_threads(1)
    try:
        with ThreadPoolExecutor(workers) as ex:
            results = list(ex.map(run, range((1 << 32) // chunk)))
    finally:
        torch.set_num_threads(threads)
    mismatches = sum(r[1] for r in results)
    assert mismatches == 0, [r[0] for r in results if r[1]][:4]
    assert all(r[2] for r in results)


def test_f32_to_f16_all_2_32_patterns():
    _all_2_32("f16", lambda x: torch.from_numpy(x).to(torch.float16).view(torch.int16)
              .numpy().view(np.uint16))


def test_f32_to_bf16_all_2_32_patterns():
    _all_2_32("bf16", _f32_to_bf16_torch)
