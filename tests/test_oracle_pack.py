"""Pins of the oracle's int4 container (section 06 of the reader.mx article
"惊呆了！25GB 内存上运行 GLM 5.2 744B 模型").  CPU only."""
import os

import numpy as np
import pytest

import oracle
from ref64 import unpack64

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "unpack_example.txt")


def _golden():
    vals = {}
    for line in open(GOLDEN, encoding="utf-8"):
        if line.startswith("#") or ":" not in line:
            continue
        k, v = line.split(":", 1)
        vals[k.strip()] = v.split()
    return vals


def test_worked_example_decodes_as_printed():
    g = _golden()
    raw = np.array([int(b, 16) for b in g["bytes"]], np.uint8)[None, :]
    q = oracle.unpack_int4(raw, 16)[0]
    assert q[0::2].tolist() == [int(v) for v in g["low_nibble_values"]]
    # the odd columns sit in the high hex digit of each printed byte
    assert q[1::2].tolist() == [int(b[0], 16) - 8 for b in g["bytes"]]


def test_worked_example_size_identity():
    g = _golden()
    rows, cols, nbytes = int(g["rows"][0]), int(g["cols"][0]), int(g["nbytes"][0])
    q4, s = oracle.pack_int4(np.ones((2, cols), np.float32))
    assert q4.shape == (2, cols // 2) and s.shape == (2,)
    assert rows * q4.shape[1] == nbytes


def test_expert_bytes_about_19mb():
    # gate/up [2048][6144] and down [6144][2048] packed, plus float row scales
    row_gu = oracle.pack_int4(np.ones((1, 6144), np.float32))[0].shape[1]
    row_d = oracle.pack_int4(np.ones((1, 2048), np.float32))[0].shape[1]
    total = 2 * 2048 * row_gu + 6144 * row_d + 4 * (2 * 2048 + 6144)
    assert total == 18_915_328  # "about 19 MB" (section 01), "18.9 MB" (section 13)


def test_unpack_then_pack_roundtrip_every_byte():
    # every byte whose nibbles are both in 1..15 (values -7..7) survives
    # unpack -> scale by a power of two -> pack; a trailing 0xFF holds a 7 so
    # that amax/7 is that power of two exactly
    bytes_ok = np.array([b for b in range(256) if (b & 15) and (b >> 4)] + [0xFF], np.uint8)[None, :]
    C = 2 * bytes_ok.shape[1]
    q = oracle.unpack_int4(bytes_ok, C).astype(np.float32)
    for k in (0, 3, 10):
        q4, s = oracle.pack_int4(q * np.float32(2.0 ** -k))
        assert s[0] == np.float32(2.0 ** -k)
        assert np.array_equal(q4, bytes_ok)


def test_nibble_layout_matches_independent_reader():
    rng = np.random.default_rng(1)
    q4 = rng.integers(0, 256, size=(5, 37), dtype=np.uint8)
    for C in (73, 74):
        assert np.array_equal(oracle.unpack_int4(q4, C).astype(np.int64), unpack64(q4, C))


def test_pack_closed_form_power_of_two_scale():
    rng = np.random.default_rng(2)
    q = rng.integers(-7, 8, size=(6, 40)).astype(np.float32)
    q[:, 5] = 7
    q[::2, 5] = -7
    scales = np.float32(2.0) ** -np.arange(6, dtype=np.float32)
    w = q * scales[:, None]
    q4, s = oracle.pack_int4(w)
    assert np.array_equal(s, scales)
    assert np.array_equal(oracle.unpack_int4(q4, 40), q.astype(np.int8))


def test_pack_rounds_half_to_even():
    w = np.array([[7.0, 2.5, 3.5, -2.5, -3.5, 0.5, 1.5, -0.5, 6.5, -6.5]], np.float32)
    q4, s = oracle.pack_int4(w)
    assert s[0] == 1.0
    assert oracle.unpack_int4(q4, 10)[0].tolist() == [7, 2, 4, -2, -4, 0, 2, 0, 6, -6]


def test_pack_never_emits_minus_eight_and_error_bound():
    rng = np.random.default_rng(3)
    w = (rng.standard_normal((64, 301)) * 0.02).astype(np.float32)
    q4, s = oracle.pack_int4(w)
    q = oracle.unpack_int4(q4, 301)
    assert q.min() >= -7 and q.max() <= 7  # |w|/s <= 7 by construction of s
    assert np.all(np.abs(q).max(axis=1) == 7)
    err = np.abs(q.astype(np.float64) * s[:, None] - w)
    assert np.all(err <= 0.5 * s[:, None] * (1 + 1e-6))


def test_pack_zero_row_and_odd_pad():
    q4, s = oracle.pack_int4(np.zeros((1, 5), np.float32))
    assert s[0] == np.float32(1e-8)
    assert q4.tolist() == [[0x88, 0x88, 0x88]]
    q4, _ = oracle.pack_int4(np.array([[7.0, -7.0, 7.0]], np.float32))
    assert q4[0, 1] == (8 + 7) | (8 << 4)  # the odd last column pads with nibble 8


def test_pack_agrees_with_vectorized_numpy_quantizer():
    """Section 07 reports that the Python converter (numpy rint) and the C
    packer (lrintf) write identical bytes.  An independent vectorized numpy
    version of the section 06 converter must match the oracle byte for byte."""
    rng = np.random.default_rng(4)
    w = (rng.standard_normal((200, 512)) * 0.02).astype(np.float32)
    amax = np.abs(w).max(axis=1, keepdims=True)
    s = np.maximum(amax / np.float32(7), np.float32(1e-8)).astype(np.float32)
    q = np.clip(np.rint(w / s), -8, 7).astype(np.int32)
    ref = ((q[:, 0::2] + 8) | ((q[:, 1::2] + 8) << 4)).astype(np.uint8)
    q4, so = oracle.pack_int4(w)
    assert np.array_equal(so, s[:, 0])
    assert np.array_equal(q4, ref)


@pytest.mark.parametrize("bad", [(0, 4), (3, 0)])
def test_pack_rejects_bad_shapes(bad):
    lib = oracle.lib()
    buf = np.zeros(16, np.float32)
    out = np.zeros(16, np.uint8)
    assert lib.moe_ref_pack_int4(buf.ctypes.data, bad[0], bad[1], out.ctypes.data,
                                 buf.ctypes.data) != 0
