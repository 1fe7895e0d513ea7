"""The benchmark's algorithmic bytes (the numerator of every GB/s figure it
reports) against closed forms worked out by hand from the unit counts, the
seeded routings they are computed from, and its single-GPU refusal."""
import os
import subprocess
import sys

import numpy as np

import bench
import synthetic_inputs as si

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_prefill_bytes_closed_form():
    # scatter: 8192 token rows of 2 * 7168 B read; 65536 rows of 7168 fp8
    # bytes and 56 scale bytes written; the 8192 x 8 int32 index table
    assert bench.bytes_scatter(8192, 8192, 8, 7168, 128, 65536) == (
        117_440_512 + 469_762_048 + 3_670_016 + 262_144)
    assert bench.bytes_scatter(8192, 8192, 8, 7168, 128, 65536) == 591_134_720
    # combine: 65536 expert rows of 2 * 7168 B read; index + weight tables;
    # 8192 bf16 output rows
    assert bench.bytes_combine(8192, 8, 7168, 65536) == (
        939_524_096 + 524_288 + 117_440_512)
    assert bench.bytes_combine(8192, 8, 7168, 65536) == 1_057_488_896
    # layout: ids read, src2dst written, m_indices over 98048 rows, counts,
    # masked_m and 257 region starts
    assert bench.bytes_layout(8192, 8, 256, 98048) == (
        262_144 + 262_144 + 392_192 + 2048 + 1028)
    assert bench.bytes_layout(8192, 8, 256, 98048) == 919_556


def test_large_combine_bytes_closed_form():
    # 131072 rows of 2 * 4096 B, 16384 x 8 index + weight entries, 16384
    # bf16 rows out
    assert bench.bytes_combine(16384, 8, 4096, 131072) == 1_209_008_128


def test_prefill_routing_counts():
    """Every assignment of the prefill routing is local and every token has
    a destination, so the step's bytes use 65536 assignments and 8192
    tokens; some experts receive nothing."""
    b = si.prefill_compact()
    ids = b.topk_ids
    assert ids.shape == (8192, 8)
    local = (ids >= 0) & (ids < b.n_local)
    assert int(local.sum()) == 65536
    assert int(local.any(axis=1).sum()) == 8192
    counts = np.bincount(ids.ravel(), minlength=b.n_local)
    assert (counts == 0).any()


def test_decode_bytes_from_its_routing():
    """The decode row's bytes come from the seeded routing: local
    assignments of experts [0, 32) and the tokens that have one."""
    b = si.decode_masked()
    local = (b.topk_ids >= 0) & (b.topk_ids < 32)
    A = int(local.sum())
    touched = int(local.any(axis=1).sum())
    want = touched * 2 * 7168 + A * (7168 + 56) + 128 * 8 * 4
    assert bench.bytes_scatter(touched, 128, 8, 7168, 128, A) == want
    assert bench.bytes_combine(128, 8, 7168, A) == (
        A * 2 * 7168 + 128 * 8 * 8 + 128 * 7168 * 2)
    # the figures the decode row reports: 140 local assignments over 89
    # tokens (39 of the 128 tokens have no local expert)
    assert (A, touched) == (140, 89)
    assert bench.bytes_scatter(touched, 128, 8, 7168, 128, A) == 2_291_360
    assert bench.bytes_combine(128, 8, 7168, A) == 3_850_240


def test_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"),
                        "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
