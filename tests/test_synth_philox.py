"""The host side of the counter-based generator (synth_philox.c), pinned to
the generator's published known-answer vectors and to the normal
distribution; the HIP library's dv_fill_normal is checked against it in the
GPU tests."""
import json
import math
import os

import numpy as np
import pytest
from scipy import stats

from contextual_sparsity_decoding_amd import synth

GOLD = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "philox_kat.json")


def test_known_answer_vectors():
    kat = json.load(open(GOLD))
    for v in kat["vectors"]:
        ctr = [int(x, 16) for x in v["counter"]]
        key = [int(x, 16) for x in v["key"]]
        want = [int(x, 16) for x in v["out"]]
        assert [int(x) for x in synth.philox_block(ctr, key)] == want


def test_words_follow_the_stream_layout():
    """Element i of stream (seed, s) is word i % 4 of the block with counter
    (i / 4, 0, s_lo, s_hi) under key (seed_lo, seed_hi)."""
    seed, s = (7 << 32) | 11, (3 << 16) | 5
    w = synth.philox_words(40, seed, s)
    for i in (0, 1, 2, 3, 4, 17, 39):
        blk = synth.philox_block([i // 4, 0, s & 0xFFFFFFFF, s >> 32], [seed & 0xFFFFFFFF, seed >> 32])
        assert w[i] == blk[i % 4]
    # a block index past 2^32 moves into the counter's second word
    b = (1 << 32) + 5
    w2 = synth.philox_words(4, seed, s, offset=4 * b)
    assert list(w2) == list(synth.philox_block([5, 1, s & 0xFFFFFFFF, s >> 32], [seed & 0xFFFFFFFF, seed >> 32]))


def test_ranges_regenerate_the_same_elements():
    full = synth.philox_normal(1003, 5, 9)
    for lo, n in ((0, 1003), (1, 10), (7, 500), (1000, 3)):
        assert np.array_equal(synth.philox_normal(n, 5, 9, offset=lo), full[lo:lo + n])
    fw = synth.philox_words(1003, 5, 9)
    assert np.array_equal(synth.philox_words(17, 5, 9, offset=13), fw[13:30])


def test_box_muller_of_the_words():
    """z for a pair (xa, xb): sqrt(-2 ln u) cos / sin (2 pi v), u = (xa + 1) / 2^32, v = xb / 2^32."""
    n = 4096
    w = synth.philox_words(n, 3, 4).astype(np.float64)
    u = (w[0::2] + 1.0) / 2.0 ** 32
    v = w[1::2] / 2.0 ** 32
    r = np.sqrt(-2.0 * np.log(u))
    want = np.empty(n)
    want[0::2] = r * np.cos(2 * np.pi * v)
    want[1::2] = r * np.sin(2 * np.pi * v)
    got = synth.philox_normal(n, 3, 4, mean=0.0, std=1.0).astype(np.float64)
    assert np.max(np.abs(got - want.astype(np.float32))) <= 1e-6
    got2 = synth.philox_normal(n, 3, 4, mean=1.5, std=0.02).astype(np.float64)
    assert np.max(np.abs(got2 - (1.5 + 0.02 * want))) <= 2e-7


def test_normal_distribution():
    z = synth.philox_normal(1 << 20, 1234, synth.stream_id(2, "w1_t")).astype(np.float64)
    assert abs(z.mean()) < 5 / math.sqrt(z.size)
    assert abs(z.var() - 1) < 0.01
    assert stats.kstest(z, "norm").pvalue > 1e-3
    # the raw words are uniform over 16 bins
    w = synth.philox_words(1 << 18, 1234, 77)
    hist = np.bincount(w >> 28, minlength=16)
    assert stats.chisquare(hist).pvalue > 1e-3


def test_streams_differ():
    a = synth.philox_words(64, 1, synth.stream_id(0, "w1_t"))
    b = synth.philox_words(64, 1, synth.stream_id(1, "w1_t"))
    c = synth.philox_words(64, 2, synth.stream_id(0, "w1_t"))
    d = synth.philox_words(64, 1, synth.stream_id(0, "w2_t"))
    assert len({a.tobytes(), b.tobytes(), c.tobytes(), d.tobytes()}) == 4


def test_half_storage_rounds_the_float():
    t = synth.philox_tensor((8, 16), 9, 3, "w1_t", 0.02, np.float16)
    f = synth.philox_normal(128, 9, synth.stream_id(3, "w1_t"), std=0.02)
    assert t.dtype == np.float16
    assert np.array_equal(t.ravel(), f.astype(np.float16))
