"""The seeded input generator: determinism, its published definition, and the
moments of the distributions it stands in for.  CPU only."""
import numpy as np

import synth

M64 = (1 << 64) - 1
GAMMA = 0x9E3779B97F4A7C15


def _mix(z):
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & M64
    return z ^ (z >> 31)


def _splitmix64_sequence(seed, n):
    state, out = seed, []
    for _ in range(n):
        state = (state + GAMMA) & M64
        out.append(_mix(state))
    return out


def test_splitmix64_published_vector():
    # first outputs of Vigna's splitmix64 seeded with 1234567
    assert _splitmix64_sequence(1234567, 5) == [
        6457827717110365317, 3203168211198807973, 9817491932198370423,
        4593380528125082431, 16408922859458223821]


def test_ih8_matches_python_definition():
    seed, strm = 11, synth.stream(synth.K_GATE, 3, 7)
    key = _mix((_mix((seed * GAMMA + 0x2545F4914F6CDD1D) & M64)) ^ _mix((strm + GAMMA) & M64))
    want = []
    for i in range(50):
        r0 = _mix((key + (2 * i + 1) * GAMMA) & M64)
        r1 = _mix((key + (2 * i + 2) * GAMMA) & M64)
        s = sum((r >> sh) & 0xFFFF for r in (r0, r1) for sh in (0, 16, 32, 48))
        want.append(s - 262140)
    assert synth.host_ih8(seed, strm, 50).tolist() == want


def test_normal_moments_and_determinism():
    a = synth.host_normal(0, synth.stream(synth.K_X), 1 << 20, 0.02)
    b = synth.host_normal(0, synth.stream(synth.K_X), 1 << 20, 0.02)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    assert abs(a.mean()) < 1e-4
    assert abs(a.std() / 0.02 - 1) < 5e-3
    c = synth.host_normal(1, synth.stream(synth.K_X), 1 << 10, 0.02)
    assert not np.array_equal(a[:1024], c)
    # a window starting mid-stream equals the same slice of the full stream
    w = synth.host_normal(0, synth.stream(synth.K_X), 100, 0.02, start=5000)
    assert np.array_equal(w, a[5000:5100])


def test_uniform_range_and_mean():
    u = synth.host_uniform(0, synth.stream(synth.K_ROUTER_B), 1 << 18, -0.1, 0.1)
    assert u.min() >= -0.1 and u.max() < 0.1
    assert abs(u.mean()) < 1e-3


def test_bf16_rounding_nearest_even():
    x = np.array([1.0, 1.00390625, 1.01171875, -2.5, 3.0e38, 1e-40], np.float32)
    bits = synth.bf16_bits(x)
    back = synth.bf16_to_f32(bits)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: even mantissa wins (1.0);
    # 1 + 3*2^-8 is a tie between 1 + 2^-7 and 1 + 2^-6: even wins (1 + 2^-6)
    assert back[0] == 1.0 and back[1] == 1.0 and back[2] == np.float32(1 + 2 ** -6)
    assert back[3] == -2.5
    r = np.random.default_rng(0).standard_normal(4096).astype(np.float32)
    rb = synth.bf16_to_f32(synth.bf16_bits(r))
    assert np.all(np.abs(rb - r) <= np.abs(r) * 2.0 ** -8)
