"""GPU parity for two data-dependent choices inside the kernel.

The start threshold over the whole ring blocks is an estimate from the first
block, confirmed by a count over those blocks; rows whose first block is not
like the next two make the count reject it (the row then starts from the
first block's own bound), on one workgroup per row and on shared rows.

A workgroup with a short share of a row may instead start from an estimate
of the row's fk-th largest value (f = 1.5, 2 or 3 by shape), read from its
first block and accepted when the ring's count agrees.  On a shared row the merge then checks that at
least k merged candidates lie above the row's largest estimate; on a row
with one workgroup the stream must end with at least k candidates.  Either
way the row is read again when the check fails.  Rows whose (first)
workgroup sees only large values in its ring make the check fail; rows whose
first block alone is large make the ring refuse the estimate.

The epilogue sort ranks small bins directly but splits bins of 9..32 members
again when ranking them would cost more than another level; bf16 rows with a
few dozen copies of each value among the results take that path, rows with
small tie groups the other.  Either way the result is the oracle's, bit for
bit.
"""
from __future__ import annotations

import numpy as np
import pytest

import workloads
from tests.gpu_util import BF16, FP32, check_case

pytestmark = pytest.mark.gpu

B = 4096   # elements per block


def _blocky_rows(nblocks: int, big_every: int, seed: int, batch: int = 3) -> np.ndarray:
    """Rows of nblocks whole blocks: block b holds 100 + U[0,1) when b is a
    multiple of big_every, else U[0,1)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    x = rng.random((batch, nblocks * B), dtype=np.float32)
    for b in range(0, nblocks, big_every):
        x[:, b * B:(b + 1) * B] += np.float32(100.0)
    return x


@pytest.mark.parametrize("plan", [
    {"segments": 1, "in_order": 1, "kernel": 1},   # ring 0,1,2: big, small, small -> estimate rejected
    {"segments": 2, "in_order": 1, "kernel": 1},   # one workgroup rejects, the other confirms
    {"segments": 3, "in_order": 1, "kernel": 1},
    {"segments": 1, "kernel": 1},                  # random order: either outcome
])
@pytest.mark.parametrize("k", [1024, 2048])
def test_start_estimate_rejected_or_confirmed_fp32(plan, k):
    x = _blocky_rows(16, 4, seed=31 + k)
    check_case(x, FP32, x.shape[1], k, 1, True, "int32", plan=plan,
               name=f"blocky fp32 k={k} {plan}")


@pytest.mark.parametrize("plan", [{"segments": 1, "in_order": 1, "kernel": 1}, {"segments": 2, "in_order": 1, "kernel": 1}])
def test_start_estimate_rejected_bf16(plan):
    x = workloads.to_bf16_bits(_blocky_rows(12, 3, seed=41))
    check_case(x, BF16, x.shape[1], 512, 0, False, "int32", plan=plan,
               name=f"blocky bf16 k=512 {plan}")
    check_case(x, BF16, x.shape[1], 512, 1, True, "int64", plan=plan,
               name=f"blocky bf16 k=512 sorted {plan}")


def _hot_blocks(nblocks: int, hot, seed: int, batch: int = 3) -> np.ndarray:
    """Rows of nblocks whole blocks of U[0,1), plus 100 in the blocks `hot`."""
    rng = np.random.Generator(np.random.PCG64(seed))
    x = rng.random((batch, nblocks * B), dtype=np.float32)
    for b in hot:
        x[:, b * B:(b + 1) * B] += np.float32(100.0)
    return x


# In block order, workgroup 0 of S reads blocks 0, S, 2S, ... and its ring holds
# the first three.  All three large: its estimate (the 2kB/L-th largest of block
# 0, about the 65th at k = 1024 and 32 blocks) is accepted, but only about 200
# elements of the row lie above it, so the merge reads the row again.
@pytest.mark.parametrize("segments", [4, 8])
@pytest.mark.parametrize("k", [512, 1024])
def test_start_estimate_fails_merge_check_fp32(segments, k):
    x = _hot_blocks(32, (0, segments, 2 * segments), seed=53 + segments + k)
    plan = {"segments": segments, "in_order": 1, "kernel": 1}
    check_case(x, FP32, x.shape[1], k, 1, True, "int64", plan=plan,
               name=f"hot ring fp32 k={k} S={segments}")
    check_case(x, FP32, x.shape[1], k, 0, False, "int32", plan=plan,
               name=f"hot ring fp32 unsorted k={k} S={segments}")
    check_case(x, FP32, x.shape[1], k, 2, False, "int32", plan=plan,
               name=f"hot ring fp32 by column k={k} S={segments}")


def test_start_estimate_fails_merge_check_ragged_and_end():
    """The row read again ends in a partial block (n_cols and end)."""
    x = _hot_blocks(32, (0, 8, 16), seed=59)
    n = x.shape[1] - 1000
    plan = {"segments": 8, "in_order": 1, "kernel": 1}
    check_case(x[:, :n].copy(), FP32, n, 1024, 1, True, "int32", plan=plan,
               name="hot ring fp32 ragged")
    end = np.array([n, x.shape[1], x.shape[1] - 4096 - 7], dtype=np.int32)
    check_case(x, FP32, x.shape[1], 1024, 1, True, "int32", end=end, plan=plan,
               name="hot ring fp32 end")


def test_start_estimate_fails_merge_check_bf16():
    # 1 + U[0,1) in the large blocks and U[0,1)/4 elsewhere: bf16 keeps 128
    # levels in [1, 2), fine enough for the estimate to sit above the k-th
    rng = np.random.Generator(np.random.PCG64(61))
    x = rng.random((3, 32 * B), dtype=np.float32) * np.float32(0.25)
    for b in (0, 4, 8):
        x[:, b * B:(b + 1) * B] = np.float32(1.0) + rng.random((3, B), dtype=np.float32)
    x = workloads.to_bf16_bits(x)
    plan = {"segments": 4, "in_order": 1, "kernel": 1}
    check_case(x, BF16, x.shape[1], 512, 0, False, "int32", plan=plan,
               name="hot ring bf16 k=512")
    check_case(x, BF16, x.shape[1], 512, 1, True, "int32", plan=plan,
               name="hot ring bf16 k=512 sorted")


# One workgroup per row: the ring (blocks 0, 1, 2 in block order) all large,
# the rest small.  The estimate (the 2kB/L-th largest of block 0) is accepted,
# but fewer than k elements of the row lie above it, so the workgroup ends
# its stream with fewer than k candidates and reads the row again from t0.
@pytest.mark.parametrize("k", [1024, 2048])
def test_start_estimate_fails_final_count_one_workgroup(k):
    x = _hot_blocks(16, (0, 1, 2), seed=71 + k)
    plan = {"segments": 1, "in_order": 1, "kernel": 1}
    check_case(x, FP32, x.shape[1], k, 1, True, "int32", plan=plan,
               name=f"hot ring one wg fp32 k={k}")
    check_case(x, FP32, x.shape[1], k, 0, False, "int64", plan=plan,
               name=f"hot ring one wg fp32 unsorted k={k}")
    n = x.shape[1] - 1000   # the re-read ends in a partial block
    check_case(x[:, :n].copy(), FP32, n, k, 1, True, "int32", plan=plan,
               name=f"hot ring one wg fp32 ragged k={k}")


def test_start_estimate_fails_final_count_one_workgroup_bf16():
    rng = np.random.Generator(np.random.PCG64(73))
    x = rng.random((3, 16 * B), dtype=np.float32) * np.float32(0.25)
    for b in (0, 1, 2):
        x[:, b * B:(b + 1) * B] = np.float32(1.0) + rng.random((3, B), dtype=np.float32)
    x = workloads.to_bf16_bits(x)
    plan = {"segments": 1, "in_order": 1, "kernel": 1}
    check_case(x, BF16, x.shape[1], 2048, 1, True, "int32", plan=plan,
               name="hot ring one wg bf16 k=2048")
    check_case(x, BF16, x.shape[1], 1024, 2, False, "int32", plan=plan,
               name="hot ring one wg bf16 by column k=1024")


# Only block 0 large: the ring's count (about 65 in three blocks) scales to
# far fewer than 1.5k for the row, so workgroup 0 starts from block 0's own
# k-th largest, a valid bound.
@pytest.mark.parametrize("dtype", [FP32, BF16])
def test_start_estimate_refused_by_ring(dtype):
    x = _hot_blocks(32, (0,), seed=67)
    if dtype == BF16:
        x = workloads.to_bf16_bits(x)
    plan = {"segments": 8, "in_order": 1, "kernel": 1}
    check_case(x, dtype, x.shape[1], 1024, 1, True, "int32", plan=plan,
               name=f"hot block 0 {'bf16' if dtype else 'fp32'}")


# k above half a block: the start is the k-th largest of the first three
# whole blocks (a valid bound), for one workgroup per row and for shares of
# four blocks; normal rows and rows whose ring blocks are all large.
@pytest.mark.parametrize("k", [2049, 3000, 4096])
@pytest.mark.parametrize("dtype", [FP32, BF16])
@pytest.mark.parametrize("segments", [1, 4])
def test_three_block_start_large_k(k, dtype, segments):
    rng = np.random.Generator(np.random.PCG64(k + segments))
    f = rng.standard_normal((3, 16 * B)).astype(np.float32)
    x = workloads.to_bf16_bits(f) if dtype == BF16 else f
    plan = {"segments": segments, "kernel": 1}
    check_case(x, dtype, 16 * B, k, 1, True, "int32", plan=plan,
               name=f"three-block start k={k} S={segments}")
    h = _hot_blocks(16, (0, segments, 2 * segments), seed=k)
    h = workloads.to_bf16_bits(h) if dtype == BF16 else h
    check_case(h, dtype, 16 * B, k, 0, False, "int32", plan={"segments": segments, "in_order": 1, "kernel": 1},
               name=f"three-block start, large ring k={k} S={segments}")


def _levels_bf16(batch: int, n: int, levels: int, seed: int) -> np.ndarray:
    """bf16 rows (as bits) taking `levels` consecutive bf16 codes from 1.0 up,
    so `levels` distinct values, each about n / levels times."""
    rng = np.random.Generator(np.random.PCG64(seed))
    lv = rng.integers(0, levels, size=(batch, n))
    return (0x3F80 + lv).astype(np.uint16)


@pytest.mark.parametrize("levels,k", [
    (2048, 2048),   # about 32 copies of each value among the results: bins split again
    (8192, 1024),   # about 8 copies: bins ranked directly
    (64, 512),      # about 1024 copies: bins larger than any rank limit
])
@pytest.mark.parametrize("segments", [1, 4])
def test_sort_with_tie_groups(levels, k, segments):
    x = _levels_bf16(4, 65536, levels, seed=levels + k)
    check_case(x, BF16, 65536, k, 1, True, "int32", plan={"segments": segments, "kernel": 1},
               name=f"ties levels={levels} k={k} S={segments}")
    check_case(x, BF16, 65536, k, 2, False, "int32", plan={"segments": segments, "kernel": 1},
               name=f"ties by column levels={levels} k={k} S={segments}")


# The merge's exact cut of a small buffer (at most a few per thread): one
# histogram finds the boundary bin, whose members are ranked directly, or
# kept whole when all of them are needed; a boundary bin of more than 64
# members (heavy bf16 ties) goes the general way.  Unsorted results on
# shared rows take it; rows barely longer than k leave the merge no more
# than k candidates.
@pytest.mark.parametrize("segments", [2, 4])
@pytest.mark.parametrize("k", [64, 512])
def test_merge_small_cut(segments, k):
    rng = np.random.Generator(np.random.PCG64(101 + k + segments))
    f = rng.standard_normal((4, 16 * B)).astype(np.float32)
    plan = {"segments": segments, "kernel": 1}
    check_case(f, FP32, 16 * B, k, 0, True, "int32", plan=plan,
               name=f"small cut fp32 k={k} S={segments}")
    check_case(workloads.to_bf16_bits(f), BF16, 16 * B, k, 0, True, "int32", plan=plan,
               name=f"small cut bf16 k={k} S={segments}")
    for levels in (64, 8192):   # tie groups of about 1000 and about 8 values
        x = _levels_bf16(4, 16 * B, levels, seed=levels + k)
        check_case(x, BF16, 16 * B, k, 0, False, "int32", plan=plan,
                   name=f"small cut ties levels={levels} k={k} S={segments}")
    end = np.array([k + 1, k + 70, 2 * B + 5, 16 * B], dtype=np.int32)
    check_case(f, FP32, 16 * B, k, 0, True, "int64", end=end, plan=plan,
               name=f"small cut short rows k={k} S={segments}")


# A shared row's workgroup whose buffer ends between k + 64 and four
# candidates per thread takes its hand-over threshold from the same 256-bin
# histogram as its bound x_w (the edge of the bin holding the k-th
# candidate), or cuts the general way when that bin would overfill the
# hand-over.  Workgroup 1 of 4 (blocks 1, 5, 9, 13 in order) estimates its
# start from a normal block 1 while its other blocks sit 0.5 higher, so it
# ends with roughly 650-900 candidates; bf16 ties exercise the fallback.
@pytest.mark.parametrize("sorted_mode", [0, 1])
@pytest.mark.parametrize("dtype", [FP32, BF16])
def test_local_bin_edge_threshold(sorted_mode, dtype):
    rng = np.random.Generator(np.random.PCG64(211 + sorted_mode))
    f = rng.standard_normal((4, 16 * B)).astype(np.float32)
    for b in (5, 9, 13):
        f[:, b * B:(b + 1) * B] += np.float32(0.5)
    x = workloads.to_bf16_bits(f) if dtype == BF16 else f
    plan = {"segments": 4, "in_order": 1, "kernel": 1}
    check_case(x, dtype, 16 * B, 512, sorted_mode, True, "int32", plan=plan,
               name=f"local bin edge {'bf16' if dtype else 'fp32'} sorted={sorted_mode}")
    levels = _levels_bf16(4, 16 * B, 256, seed=7 + sorted_mode)
    check_case(levels, BF16, 16 * B, 512, sorted_mode, False, "int32", plan=plan,
               name=f"local bin edge ties sorted={sorted_mode}")


# Rows that are mostly zeros of both signs (and a few -inf), so the start's
# edges and the ring's count land on zero: the count compares values
# against the value of the edge's key, and both zeros share one key, so
# -0.0 and +0.0 must count alike; -inf must never count above a finite edge.
@pytest.mark.parametrize("segments", [1, 2])
@pytest.mark.parametrize("sorted_mode", [0, 1])
@pytest.mark.parametrize("dtype", [FP32, BF16])
def test_start_on_signed_zeros(segments, sorted_mode, dtype):
    rng = np.random.Generator(np.random.PCG64(307 + 2 * segments + sorted_mode))
    n = 8 * B
    f = np.where(rng.random((3, n)) < 0.5, np.float32(0.0), np.float32(-0.0)).astype(np.float32)
    pos = rng.random((3, n)) < 0.03
    f[pos] = np.abs(rng.standard_normal(int(pos.sum()))).astype(np.float32) + np.float32(0.5)
    f[rng.random((3, n)) < 0.01] = -np.inf
    x = workloads.to_bf16_bits(f) if dtype == BF16 else f
    for k in (256, 1024, 2048):
        check_case(x, dtype, n, k, sorted_mode, True, "int32", plan={"segments": segments, "kernel": 1},
                   name=f"signed zeros k={k} S={segments} sorted={sorted_mode}")
