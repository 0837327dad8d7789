"""Pins for the seeded input generator (CPU only)."""
import json
import os

import numpy as np

import synth
from synth import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_splitmix64_published_vectors():
    with open(os.path.join(GOLDEN, "splitmix64_vectors.json")) as f:
        ref = json.load(f)
    assert synth.splitmix64_outputs(ref["seed"], 5) == ref["outputs"]


def test_counter_form_matches_sequential_stream():
    key = 0x0123456789ABCDEF
    seq = synth.splitmix64_outputs(key, 100)
    got = synth.counter_bits(key, np.arange(100, dtype=np.uint64))
    assert [int(x) for x in got] == seq


def test_normal_table_shape_and_moments():
    tab = synth.normal_table_f32().astype(np.float64)
    assert tab.shape == (65536,)
    assert np.all(np.diff(tab) > 0)
    # symmetric quantiles
    assert np.max(np.abs(tab + tab[::-1])) < 1e-6
    assert abs(tab.mean()) < 1e-7
    assert abs((tab ** 2).mean() - 1.0) < 1e-3


def test_bf16_rounding_known_patterns():
    vals = np.array([1.0, -2.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 3.0], dtype=np.float32)
    bits = synth.f32_to_bf16_bits(vals)
    # 1+2^-8 ties to even (0x3F80); 1+3*2^-8 ties to even (0x3F82)
    assert bits.tolist() == [0x3F80, 0xC000, 0x3F80, 0x3F82, 0x4040]


def test_bf16_table_is_rounded_f32_table():
    f = synth.normal_table_f32()
    b = synth.normal_table_bf16()
    widened = (b.astype(np.uint32) << 16).view(np.float32)
    # nearest: error at most half a bf16 ulp (2^-8 relative)
    rel = np.abs(widened.astype(np.float64) - f) / np.abs(f).astype(np.float64)
    assert rel.max() <= 2.0 ** -8


def test_normals_deterministic_and_addressable():
    key = synth.stream_key(7, synth.TAG_Q, 3)
    a = synth.normals(key, 1000, 500, "f32")
    b = synth.normals_at(key, np.arange(1000, 1500, dtype=np.uint64), "f32")
    assert np.array_equal(a, b)
    c = synth.normals(key, 0, 200000, "f32").astype(np.float64)
    assert abs(c.mean()) < 0.01 and abs(c.std() - 1) < 0.01


def test_shuffle_is_permutation():
    p = synth.shuffle(synth.stream_key(3, synth.TAG_SHUFFLE), 4096)
    assert sorted(p.tolist()) == list(range(4096))
    assert not np.array_equal(p, np.arange(4096))


def test_workload_recipes():
    w2 = workloads.batch32_fp32()
    assert (w2.n, w2.layers, w2.heads, w2.head_width, w2.page_size, w2.num_pages) == \
        (32, 12, 12, 64, 16, 4096)
    assert w2.lengths.min() >= 1 and w2.lengths.max() <= 1024
    used = w2.page_tables[w2.page_tables >= 0]
    assert len(np.unique(used)) == len(used) == workloads.expected_pages(w2.lengths, 16)
    w3 = workloads.batch256_bf16()
    assert w3.lengths.min() >= 512 and w3.lengths.max() <= 4096
    w4 = workloads.skewed64_bf16()
    assert w4.lengths.min() >= 16 and w4.lengths.max() <= 32768
    assert w4.lengths.max() > 8 * w4.lengths.min()
    w5 = workloads.fullstep128_bf16()
    assert w5.lengths.min() >= 1537 and w5.lengths.max() <= 2561
    ab = np.stack([w5.abort_layer(s) for s in range(200)])
    frac = (ab >= 0).mean()
    assert 0.005 < frac < 0.015
    assert ab.max() < 32
