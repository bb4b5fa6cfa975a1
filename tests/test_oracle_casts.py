"""Pins of the oracle's 16-bit widening and round-to-nearest-even against torch's
CPU casts (a library routine independent of the oracle)."""
import numpy as np
import pytest
import torch

from oracle import casts as C


def _torch_round(x32: np.ndarray, dt) -> np.ndarray:
    return torch.from_numpy(x32).to(dt).view(torch.int16).numpy().view(np.uint16)


def _torch_widen(bits: np.ndarray, dt) -> np.ndarray:
    return torch.from_numpy(bits.view(np.int16)).view(dt).to(torch.float32).numpy()


def _same(a_bits, b_bits, nan_a, nan_b):
    """Bit-exact, except that any NaN matches any NaN."""
    return np.all(np.where(nan_a | nan_b, nan_a == nan_b, a_bits == b_bits))


def _stratified_f32() -> np.ndarray:
    """Every sign and exponent, with fraction patterns around both formats'
    rounding boundaries (halfway, halfway +- 1 ulp, odd/even kept bit) and random
    fractions."""
    rng = np.random.default_rng(1234)
    fr = [0, 1, 2, 0x7FFFFF, 0x7FFFFE, 0x400000, 0x3FFFFF]
    for keep in (7, 10):
        half = 1 << (22 - keep)
        for kept in (0, 1, 2, 3, (1 << keep) - 1, (1 << keep) - 2):
            base = kept << (23 - keep)
            fr += [base + half - 1, base + half, base + half + 1, base, base + 1,
                   base + (1 << (23 - keep)) - 1]
    fr = np.array(sorted(set(f & 0x7FFFFF for f in fr)), dtype=np.uint32)
    rand = rng.integers(0, 1 << 23, size=512, dtype=np.uint32)
    fracs = np.concatenate([fr, rand])
    e = np.arange(256, dtype=np.uint32)
    s = np.array([0, 1], dtype=np.uint32)
    bits = (s[:, None, None] << 31) | (e[None, :, None] << 23) | fracs[None, None, :]
    return bits.reshape(-1).view(np.float32)


def test_widen_f16_exhaustive():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    a = C.widen_f16(bits)
    b = _torch_widen(bits, torch.float16)
    assert _same(a.view(np.uint32), b.view(np.uint32), np.isnan(a), np.isnan(b))


def test_widen_bf16_exhaustive():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    a = C.widen_bf16(bits)
    b = _torch_widen(bits, torch.bfloat16)
    assert _same(a.view(np.uint32), b.view(np.uint32), np.isnan(a), np.isnan(b))


@pytest.mark.parametrize("fmt", ["bf16", "f16"])
def test_round_stratified(fmt):
    x = _stratified_f32()
    ours = C.round_to_bf16(x) if fmt == "bf16" else C.round_to_f16(x)
    dt = torch.bfloat16 if fmt == "bf16" else torch.float16
    ref = _torch_round(x, dt)
    wid = C.widen_bf16 if fmt == "bf16" else C.widen_f16
    assert _same(ours, ref, np.isnan(wid(ours)), np.isnan(wid(ref)))


def test_round_known_values():
    """Hand-checked cases: ties to even, overflow at fp16's max + half an ulp,
    subnormals, signed zero."""
    f = np.float32
    x = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8, 65504.0, 65519.0, 65520.0, 2.0**-24,
                  2.0**-25, 1.5 * 2.0**-25, -0.0], dtype=f)
    bf = C.round_to_bf16(x)
    h = C.round_to_f16(x)
    # bf16: 1 + 2^-8 is a tie between 1 and 1 + 2^-7 -> even (1.0); 1 + 3*2^-8 -> 1 + 2^-6
    assert bf[0] == 0x3F80 and bf[1] == 0x3F80 and bf[2] == 0x3F82
    # fp16: 65504 max finite; 65519 stays; 65520 is the tie with 65536 -> inf
    assert h[3] == 0x7BFF and h[4] == 0x7BFF and h[5] == 0x7C00
    # fp16 subnormals: 2^-24 is the smallest; 2^-25 ties to 0 (even); 1.5*2^-25 -> 2^-24
    assert h[6] == 0x0001 and h[7] == 0x0000 and h[8] == 0x0001
    assert h[9] == 0x8000 and bf[9] == 0x8000


@pytest.mark.slow
@pytest.mark.parametrize("fmt", ["bf16", "f16"])
def test_round_exhaustive(fmt):
    """All 2^32 fp32 bit patterns (ZERO_EXHAUSTIVE=1; a few minutes)."""
    dt = torch.bfloat16 if fmt == "bf16" else torch.float16
    rnd = C.round_to_bf16 if fmt == "bf16" else C.round_to_f16
    wid = C.widen_bf16 if fmt == "bf16" else C.widen_f16
    step = 1 << 24
    for lo in range(0, 1 << 32, step):
        x = np.arange(lo, lo + step, dtype=np.uint64).astype(np.uint32).view(np.float32)
        a, b = rnd(x), _torch_round(x, dt)
        assert _same(a, b, np.isnan(wid(a)), np.isnan(wid(b))), hex(lo)


def test_widen_dispatch():
    x = np.array([1.5, -2.0], dtype=np.float32)
    assert np.array_equal(C.widen(x, "f32"), x)
    assert np.array_equal(C.widen(C.narrow(x, "bf16"), "bf16"), x)
    assert np.array_equal(C.widen(C.narrow(x, "f16"), "f16"), x)
    with pytest.raises(ValueError):
        C.widen(x, "f8")
