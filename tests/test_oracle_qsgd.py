"""Pins for the oracle's b-bit stochastic quantizer, b in {2, 4, 8} (CPU only).

SparCML §6 (QSGD with 2-, 4- and 8-bit outputs: buckets quantized
independently and stochastically, one full-precision scale each), §2.2
(zero-mean noise) and §4 (the reduced dense vector may be quantized). The
codes are unpacked here with plain numpy bit operations, independently of
the oracle, and checked against invariants, hand-packed bytes, unbiasedness
over many seeds and a recomputation from rocRAND's Philox stream.
"""
import subprocess

import numpy as np
import pytest

import oracle

LEVELS = {2: 1, 4: 7, 8: 127}


def _unpack(codes, n, bits):
    """[P, ceil(n*bits/8)] u8 -> (level, sign) [P, n]; position e sits at bit
    (e mod 8/bits)*bits of byte e*bits/8."""
    per = 8 // bits
    e = np.arange(n)
    raw = (codes[:, e // per].astype(np.uint32) >> ((e % per) * bits).astype(np.uint32)) & ((1 << bits) - 1)
    return raw & LEVELS[bits], raw >> (bits - 1)


@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("n,bucket", [(1, 8), (7, 8), (13, 8), (1000, 512), (1311, 512), (4097, 1024)])
def test_shapes_scale_levels_signs_spare_bits(bits, n, bucket):
    rng = np.random.default_rng(n * 10 + bits)
    P = 3
    v = (rng.standard_normal((P, n)) * 1e-3).astype(np.float32)
    codes, scales = oracle.qsgd(v, bits, bucket, seed=77, step=2)
    nb = -(-n // bucket)
    assert codes.shape == (P, -(-n * bits // 8)) and scales.shape == (P, nb)
    for p in range(P):
        for j in range(nb):
            assert scales[p, j] == np.abs(v[p, j * bucket:(j + 1) * bucket]).max()
    level, sign = _unpack(codes, n, bits)
    assert np.all(level <= LEVELS[bits])
    np.testing.assert_array_equal(sign, (v < 0).astype(np.uint32))
    used = n * bits % 8
    if used:  # bits past the last position stay zero
        assert np.all(codes[:, -1] >> used == 0)


def test_hand_packed_bytes():
    """Deterministic levels (|v| = scale -> s, v = 0 -> 0) packed by hand."""
    v = np.array([[2.0, 0.0, -2.0, -0.0, 0.0, 2.0, -2.0, 0.0]], np.float32)
    c2, s2 = oracle.qsgd(v, 2, 8, seed=1, step=0)
    # codes 01 00 11 00 | 00 01 11 00, lowest position in the lowest bits
    assert s2.tolist() == [[2.0]]
    assert c2.tolist() == [[0b00110001, 0b00110100]]
    c8, _ = oracle.qsgd(v, 8, 8, seed=1, step=0)
    assert c8.tolist() == [[0x7F, 0x00, 0xFF, 0x00, 0x00, 0x7F, 0xFF, 0x00]]
    c4, _ = oracle.qsgd(v, 4, 8, seed=1, step=0)
    assert c4.tolist() == [[0x07, 0x0F, 0x70, 0x0F]]


@pytest.mark.parametrize("bits", [2, 8])
def test_extremes_and_zero_bucket(bits):
    s = LEVELS[bits]
    v = np.zeros((1, 24), np.float32)
    v[0, :16] = np.linspace(-3, 3, 16).astype(np.float32)
    v[0, 20] = -0.0
    codes, scales = oracle.qsgd(v, bits, 16, seed=5, step=0)
    level, sign = _unpack(codes, 24, bits)
    assert level[0, 0] == s and sign[0, 0] == 1
    assert level[0, 15] == s and sign[0, 15] == 0
    assert scales[0, 1] == 0.0 and np.all(level[0, 16:] == 0) and np.all(sign[0, 16:] == 0)


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_dequantize_error_bound(bits):
    rng = np.random.default_rng(bits)
    n = 3000
    v = rng.laplace(0, 1e-3, size=(4, n)).astype(np.float32)
    codes, scales = oracle.qsgd(v, bits, 512, seed=4321, step=1)
    d = oracle.dqsgd(codes, scales, n, bits, 512)
    st = np.repeat(scales / np.float32(LEVELS[bits]), 512, axis=1)[:, :n]
    assert np.all(np.abs(d.astype(np.float64) - v) <= st * (1 + 1e-6) + 1e-30)
    assert np.all((d == 0) | (np.sign(d) == np.sign(v)))
    # the values the dequantizer produces are exactly +-fl32(level * fl32(scale / s))
    level, sign = _unpack(codes, n, bits)
    want = (level.astype(np.float32) * st.astype(np.float32)).astype(np.float32)
    want = np.where(sign == 1, -want, want)
    np.testing.assert_array_equal(d, want)


@pytest.mark.parametrize("bits", [2, 8])
def test_unbiased_over_seeds(bits):
    """E[dq(q(v))] = v: mean over 10^4 seeds within 5 sigma of v."""
    rng = np.random.default_rng(30 + bits)
    v = rng.standard_normal((1, 64)).astype(np.float32)
    v[0, 0] = 4.0
    S = 10000
    acc = np.zeros(64)
    for t in range(S):
        codes, scales = oracle.qsgd(v, bits, 64, seed=t * 2654435761 + 7, step=t % 5)
        acc += oracle.dqsgd(codes, scales, 64, bits, 64)[0]
    mean = acc / S
    st = np.float32(4.0) / np.float32(LEVELS[bits])
    sigma = st * 0.5 / np.sqrt(S)
    assert np.all(np.abs(mean - v[0]) <= 5 * sigma + 1e-6)


@pytest.mark.parametrize("bits", [2, 8])
def test_levels_recomputed_from_rocrand_stream(rocrand_probe, bits):
    """Row r of a call with node0 = 3 draws word (e & 3) of the block at
    counter {e>>2, 3 + r, step, 0}; the level is floor(x) + (u < frac(x))."""
    n, P, step, seed, node0 = 40, 2, 9, 0x0BAD_5EED_1234_5678, 3
    rng = np.random.default_rng(bits)
    v = rng.uniform(-1, 1, size=(P, n)).astype(np.float32)
    codes, scales = oracle.qsgd(v, bits, n, seed, step, node0=node0)
    level, _ = _unpack(codes, n, bits)
    key = [seed & 0xFFFFFFFF, seed >> 32]
    lines = [f"{b} {node0 + p} {step} 0 {key[0]} {key[1]}" for p in range(P) for b in range(n // 4)]
    out = subprocess.run([rocrand_probe], input="\n".join(lines) + "\n", capture_output=True,
                         text=True, check=True).stdout.split("\n")
    words = np.array([list(map(int, l.split())) for l in out if l.strip()], np.uint64).reshape(P, n // 4, 4)
    s = np.float32(LEVELS[bits])
    for p in range(P):
        x = ((np.abs(v[p]) / scales[p, 0]).astype(np.float32) * s).astype(np.float32)
        lo = np.floor(x)
        f = (x - lo).astype(np.float32)
        u = (words[p].reshape(-1) >> np.uint64(8)).astype(np.float32) * np.float32(2.0 ** -24)
        np.testing.assert_array_equal(level[p], lo.astype(np.int64) + (u < f))


def test_node0_names_the_counter_node():
    rng = np.random.default_rng(4)
    v = rng.standard_normal((3, 333)).astype(np.float32)
    c_all, s_all = oracle.qsgd(v, 4, 64, seed=11, step=3)
    for r in range(3):
        c_one, s_one = oracle.qsgd(v[r:r + 1], 4, 64, seed=11, step=3, node0=r)
        np.testing.assert_array_equal(c_one[0], c_all[r])
        np.testing.assert_array_equal(s_one[0], s_all[r])
