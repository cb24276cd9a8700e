"""Pins for the oracle's Philox-4x32-10 and 4-bit stochastic quantizer (CPU only).

SparCML §6 (QSGD: buckets quantized independently and stochastically with one
full-precision scale each; 2/4/8-bit outputs) and §2.2 (zero-mean
quantization noise). The Philox block is pinned against rocRAND's own engine;
the quantizer by its invariants and by unbiasedness over many seeds.
"""
import subprocess

import numpy as np
import pytest

import oracle


def test_philox_block_matches_rocrand(rocrand_probe):
    rng = np.random.default_rng(7)
    triples = [[0, 0, 0, 0, 0, 0], [1, 0, 0, 0, 0, 0], [0, 0, 0, 0, 1, 0], [0, 0, 0, 0, 0, 1],
               [0xFFFFFFFF] * 6, [5, 3, 2, 0, 0xDEADBEEF, 0x12345678]]
    triples += rng.integers(0, 2 ** 32, size=(40, 6), dtype=np.uint64).tolist()
    inp = "\n".join(" ".join(str(int(x)) for x in t) for t in triples) + "\n"
    out = subprocess.run([rocrand_probe], input=inp, capture_output=True, text=True, check=True).stdout
    ref = [list(map(int, line.split())) for line in out.strip().splitlines()]
    assert len(ref) == len(triples)
    for t, want in zip(triples, ref):
        got = oracle.philox4x32_10(t[:4], t[4:])
        assert got.tolist() == want, t


def _levels(codes, n):
    lo = codes & 0xF
    hi = codes >> 4
    both = np.stack([lo, hi], axis=-1).reshape(codes.shape[0], -1)[:, :n]
    return both & 7, both >> 3


@pytest.mark.parametrize("n,bucket", [(1, 8), (7, 8), (512, 512), (1000, 512), (1311, 512), (4097, 64)])
def test_scale_is_exact_bucket_max_and_levels_bounded(n, bucket):
    rng = np.random.default_rng(n)
    P = 3
    v = (rng.standard_normal((P, n)) * 1e-3).astype(np.float32)
    codes, scales = oracle.q4(v, bucket, seed=99, step=1)
    nb = -(-n // bucket)
    assert scales.shape == (P, nb) and codes.shape == (P, (n + 1) // 2)
    for p in range(P):
        for j in range(nb):
            assert scales[p, j] == np.abs(v[p, j * bucket:(j + 1) * bucket]).max()
    level, sign = _levels(codes, n)
    assert np.all(level <= 7)
    np.testing.assert_array_equal(sign, (v < 0).astype(np.uint8))
    if n % 2:  # the spare high nibble of an odd row stays zero
        assert np.all(codes[:, -1] >> 4 == 0)


def test_extremes_and_zero_bucket():
    v = np.zeros((2, 600), np.float32)
    v[0, :512] = np.linspace(-3, 3, 512).astype(np.float32)
    v[0, 512:] = 0.0  # all-zero partial bucket
    v[1, 3] = -0.0
    v[1, 5] = 2.5
    codes, scales = oracle.q4(v, 512, seed=5, step=0)
    level, sign = _levels(codes, 600)
    assert level[0, 0] == 7 and sign[0, 0] == 1  # |v| = scale -> level 7
    assert level[0, 511] == 7 and sign[0, 511] == 0
    assert scales[0, 1] == 0.0 and np.all(codes[0, 256:] == 0)
    assert level[1, 5] == 7
    assert np.all(level[1, [0, 1, 2, 3, 4, 6, 7]] == 0)
    assert sign[1, 3] == 0  # -0.0 is not < 0


def test_dequantize_error_bound():
    rng = np.random.default_rng(11)
    v = rng.laplace(0, 1e-3, size=(4, 3000)).astype(np.float32)
    codes, scales = oracle.q4(v, 512, seed=1234, step=3)
    d = oracle.dq4(codes, scales, 3000, 512)
    st = np.repeat(scales / np.float32(7.0), 512, axis=1)[:, :3000]
    assert np.all(np.abs(d.astype(np.float64) - v) <= st * (1 + 1e-6) + 1e-30)
    assert np.all((d == 0) | (np.sign(d) == np.sign(v)))


def test_unbiased_over_seeds():
    """E[dq4(q4(v))] = v: mean over 10^4 seeds within 5 sigma of v."""
    rng = np.random.default_rng(21)
    v = rng.standard_normal((1, 64)).astype(np.float32)
    v[0, 0] = 4.0  # fixes the scale
    S = 10000
    acc = np.zeros(64)
    for s in range(S):
        codes, scales = oracle.q4(v, 64, seed=s * 2654435761 + 1, step=s % 7)
        acc += oracle.dq4(codes, scales, 64, 64)[0]
    mean = acc / S
    st = np.float32(4.0) / np.float32(7.0)
    sigma = st * 0.5 / np.sqrt(S)
    assert np.all(np.abs(mean - v[0]) <= 5 * sigma + 1e-6)


def test_stream_depends_on_node_step_seed_and_position():
    v = np.full((2, 512), 0.35, np.float32)
    v[:, 0] = 0.7  # x = 3.5 at 0.35: level 3 or 4 with equal odds
    c0, _ = oracle.q4(v, 512, seed=1, step=0)
    c1, _ = oracle.q4(v, 512, seed=1, step=1)
    c2, _ = oracle.q4(v, 512, seed=2, step=0)
    assert not np.array_equal(c0[0], c0[1])  # node index is in the counter
    assert not np.array_equal(c0, c1)
    assert not np.array_equal(c0, c2)
    level, _ = _levels(c0, 512)
    frac4 = (level[:, 1:] == 4).mean()
    assert 0.2 < frac4 < 0.8


def test_word_selection_uses_rocrand_stream(rocrand_probe):
    """Position e draws word (e & 3) of the block at counter {e>>2, node, step, 0}."""
    n, P, step, seed = 24, 2, 5, 0x1234_5678_9ABC_DEF0
    rng = np.random.default_rng(3)
    v = rng.uniform(-1, 1, size=(P, n)).astype(np.float32)
    codes, scales = oracle.q4(v, n, seed, step)
    level, _ = _levels(codes, n)
    key = [seed & 0xFFFFFFFF, seed >> 32]
    lines = [f"{b} {p} {step} 0 {key[0]} {key[1]}" for p in range(P) for b in range(n // 4)]
    out = subprocess.run([rocrand_probe], input="\n".join(lines) + "\n", capture_output=True,
                         text=True, check=True).stdout.split("\n")
    words = np.array([list(map(int, l.split())) for l in out if l.strip()], np.uint64).reshape(P, n // 4, 4)
    for p in range(P):
        x = (np.abs(v[p]) / scales[p, 0]).astype(np.float32) * np.float32(7.0)
        x = x.astype(np.float32)
        lo = np.floor(x)
        f = (x - lo).astype(np.float32)
        u = (words[p].reshape(-1) >> np.uint64(8)).astype(np.float32) * np.float32(2.0 ** -24)
        np.testing.assert_array_equal(level[p], lo.astype(np.int64) + (u < f))
