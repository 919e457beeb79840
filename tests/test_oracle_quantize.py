"""Pins for the oracle's per-token (1x128) and per-block (128x128) quantizers.

Codes are checked against torch's float8_e4m3fn cast of the clamped ratio
(a library routine), and against invariants that hold for any correct
quantizer: the block maximum lands on code 448, signs are kept, and the
round trip is within half an e4m3 step."""
import numpy as np
import pytest
import torch


def _torch_codes(x: np.ndarray, scale_per_elem: np.ndarray) -> np.ndarray:
    r = torch.from_numpy(x) / torch.from_numpy(scale_per_elem)
    return r.clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _same_codes(a: np.ndarray, b: np.ndarray) -> bool:
    """Equal codes, treating +0 (0x00) and -0 (0x80) as one."""
    za = (a & 0x7F) == 0
    zb = (b & 0x7F) == 0
    return bool(np.array_equal(za, zb) and np.array_equal(a[~za], b[~zb]))


@pytest.mark.parametrize("M,K", [(1, 128), (7, 256), (64, 1024)])
def test_per_token_against_torch_cast(orc, M, K):
    rng = np.random.default_rng(M * 1000 + K)
    x = (rng.standard_normal((M, K)) * np.exp2(rng.integers(-8, 8, (M, 1)))).astype(np.float32)
    q, s = orc.quantize_per_token(x)
    assert q.shape == (M, K) and s.shape == (M, K // 128)
    blocks = np.abs(x).reshape(M, K // 128, 128).max(axis=2)
    assert np.array_equal(s, (torch.from_numpy(blocks) / 448.0).numpy())
    assert _same_codes(q, _torch_codes(x, np.repeat(s, 128, axis=1)))


@pytest.mark.parametrize("N,K", [(128, 128), (200, 256), (64, 384), (300, 128)])
def test_per_block_against_torch_cast(orc, N, K):
    rng = np.random.default_rng(N * 7 + K)
    x = (rng.standard_normal((N, K)) * 3).astype(np.float32)
    q, s = orc.quantize_per_block(x)
    NB, KB = (N + 127) // 128, K // 128
    assert q.shape == (N, K) and s.shape == (NB, KB)
    pad = np.zeros((NB * 128, K), dtype=np.float32)
    pad[:N] = np.abs(x)
    blocks = pad.reshape(NB, 128, KB, 128).max(axis=(1, 3))
    assert np.array_equal(s, (torch.from_numpy(blocks) / 448.0).numpy())
    per_elem = np.repeat(np.repeat(s, 128, axis=0)[:N], 128, axis=1)
    assert _same_codes(q, _torch_codes(x, per_elem))


def test_quantize_invariants(orc):
    rng = np.random.default_rng(5)
    x = rng.standard_normal((256, 512)).astype(np.float32)
    table = orc.e4m3_table()
    q_t, s_t = orc.quantize_per_token(x)
    q_b, s_b = orc.quantize_per_block(x)
    cases = [
        # (codes, per-element scale, |value| per block as [blocks][elements])
        (q_t, np.repeat(s_t, 128, axis=1),
         lambda v: np.abs(v).reshape(256, 4, 128).reshape(-1, 128)),
        (q_b, np.repeat(np.repeat(s_b, 128, axis=0), 128, axis=1),
         lambda v: np.abs(v).reshape(2, 128, 4, 128).transpose(0, 2, 1, 3).reshape(-1, 128 * 128)),
    ]
    for q, scale, blocks in cases:
        vals = table[q]
        # every block reaches the top code: amax / (amax/448) rounds to 448
        assert (blocks(vals).max(axis=1) == 448.0).all()
        # sign kept for every nonzero code
        nz = (q & 0x7F) != 0
        assert np.array_equal(np.signbit(vals[nz]), np.signbit(x[nz]))
        # round trip within half a step: e4m3 has 3 mantissa bits
        recon = vals * scale.astype(np.float64)
        normal = np.abs(x) / scale >= 2.0 ** -6
        err = np.abs(recon - x.astype(np.float64))
        assert (err[normal] <= 2.0 ** -4 * np.abs(x[normal]) * (1 + 1e-6)).all()
        sub = ~normal
        assert (err[sub] <= 2.0 ** -10 * scale[sub] * (1 + 1e-6)).all()


def test_quantize_zero_block(orc):
    x = np.zeros((3, 256), dtype=np.float32)
    x[1, 200] = -2.5
    q, s = orc.quantize_per_token(x)
    assert s[0, 0] == 0 and s[0, 1] == 0 and s[1, 0] == 0
    assert (q[0] == 0).all() and (q[1, :128] == 0).all()
    assert q[1, 200] == 0xFE and s[1, 1] == np.float32(2.5) / np.float32(448.0)
    q2, s2 = orc.quantize_per_block(np.zeros((130, 128), dtype=np.float32))
    assert (s2 == 0).all() and (q2 == 0).all()


def test_bf16_decode_pins(orc):
    """bf16 bit patterns against their values from the format's definition
    (1 sign, 8 exponent bits with bias 127, 7 fraction bits; exponent 0 is
    subnormal with 2^-126 * fraction/128)."""
    assert orc.bf16_value(0x3F80) == 1.0
    assert orc.bf16_value(0xC000) == -2.0
    assert orc.bf16_value(0x3EAA) == (1 + 42 / 128) * 2.0 ** -2
    assert orc.bf16_value(0x0001) == 2.0 ** -133
    assert orc.bf16_value(0x007F) == 127 / 128 * 2.0 ** -126
    assert orc.bf16_value(0x7F7F) == (2 - 2.0 ** -7) * 2.0 ** 127
    assert orc.bf16_value(0x7F80) == np.inf
    v = orc.bf16_value(0x8000)
    assert v == 0.0 and np.signbit(v)


def test_per_token_bf16_worked_example(orc):
    """One block by hand: amax 2 gives scale 2/448 = 1/224, so 1.0 -> 224
    (code 0x76: exponent field 14, 2^(14-7) * (1 + 6/8)), -2.0 -> -448
    (0xFE), 0.5 -> 112 (0x6E: exponent field 13), a bf16 subnormal -> 0."""
    x = np.zeros((1, 128), dtype=np.uint16)
    x[0, 0], x[0, 1], x[0, 2], x[0, 3] = 0x3F80, 0xC000, 0x3F00, 0x0001
    q, s = orc.quantize_per_token_bf16(x)
    assert s[0, 0] == np.float32(2.0) / np.float32(448.0)
    assert list(q[0, :4]) == [0x76, 0xFE, 0x6E, 0x00]
    assert (q[0, 4:] == 0).all()


def test_per_token_bf16_is_fp32_path_on_decoded_values(orc):
    rng = np.random.default_rng(16)
    bits = rng.integers(0, 1 << 16, size=(37, 384), dtype=np.uint16)
    bits[(bits & 0x7F80) == 0x7F80] = 0x3F80  # no inf/NaN inputs
    q, s = orc.quantize_per_token_bf16(bits)
    dec = (bits.astype(np.uint32) << 16).view(np.float32)
    q2, s2 = orc.quantize_per_token(dec)
    assert np.array_equal(q, q2) and np.array_equal(s, s2)
