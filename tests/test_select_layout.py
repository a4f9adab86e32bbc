"""The top-B launch plan (host logic, CPU only): fasa_select_layout reports the
layout fasa_topk / fasa_decode_step take for (max_seq_len, budget).  Exact
selection holds in every layout (the GPU parity tests check that); here each
layout's preconditions are checked over a grid, and the workloads' own shapes
are pinned to the layouts their timings were taken with."""

import itertools

import pytest

import sparse_kv_cache_rope_amd as fasa

FUSED_MAX_BUDGET = 1024   # selection and FAC share a workgroup up to this B
MAX_CANDIDATES = 16384    # the candidate stage holds at most this many

LENGTHS = [1, 2, 63, 64, 255, 256, 1000, 4095, 4096, 4097, 8191, 8192, 8193, 12000, 16383,
           16384, 16385, 20000, 24576, 32767, 32768, 32769, 32831, 40959, 40960, 40961, 65536,
           100000, 131072, 131136, 262144]
BUDGETS = [1, 2, 64, 255, 256, 257, 700, 1023, 1024, 1025, 2000, 4095, 4096, 4097, 6193, 8192,
           8193, 12000, 16384, 16385, 30000]


def candidates(n, budget, chunk):
    """Candidates of a row of n positions cut into chunks that each keep their
    own top-B: min(B, chunk) per full chunk and min(B, rest) for the last."""
    nch = -(-n // chunk)
    last = n - (nch - 1) * chunk
    return (nch - 1) * min(budget, chunk) + min(budget, last)


@pytest.mark.parametrize("n,budget", list(itertools.product(LENGTHS, BUDGETS)))
def test_layout_preconditions(n, budget):
    kind, threads, per_thread, chunk = fasa.select_layout(n, budget)
    if kind == "whole":
        assert threads in (512, 1024) and per_thread in (4, 8, 16)
        assert n <= threads * per_thread <= 16384
        assert chunk == 0
    elif kind == "chunked":
        assert chunk in (4096, 8192, 16384) and budget < chunk < n
        c = candidates(n, budget, chunk)
        assert c <= MAX_CANDIDATES and c <= threads * per_thread
        assert threads in (512, 1024) and per_thread in (4, 8, 16)
    elif kind == "whole_wide":
        assert budget > FUSED_MAX_BUDGET, "no FAC shares the 1024-thread whole-row workgroup"
        assert 16384 < n <= threads * per_thread and threads == 1024 and per_thread in (32, 40)
        assert per_thread == (32 if n <= 32768 else 40)
        assert chunk == 0
    else:
        assert kind == "per_row"
        assert n > 16384 and threads == per_thread == chunk == 0


def test_short_rows_are_held_whole():
    for n, budget in itertools.product([1, 100, 4096, 8192], BUDGETS):
        assert fasa.select_layout(n, budget)[0] == "whole"


def test_large_budgets_on_rows_chunks_barely_cut_are_held_whole():
    # 16384-position chunks would leave 12386 of 32768 positions as candidates.
    assert candidates(32768, 6193, 16384) * 4 > 32768
    assert fasa.select_layout(32768, 6193) == ("whole_wide", 1024, 32, 0)
    # Budgets that chunks do cut keep the two stages.
    assert fasa.select_layout(32768, 2000)[0] == "chunked"


def test_large_budgets_on_rows_up_to_16384_are_held_whole_16_per_thread():
    # Rows of 8193-16384 positions with B past the fused limit, where chunks
    # would leave more than a quarter of the row as candidates: one
    # 1024-thread workgroup holds the row whole, 16 scores per thread.
    for n, budget in [(9000, 2000), (12000, 2000), (16000, 8500), (16384, 4096),
                      (16384, 1025)]:
        assert fasa.select_layout(n, budget) == ("whole", 1024, 16, 0), (n, budget)
    # Budgets within the fused limit keep their chunks there.
    assert fasa.select_layout(12000, 1024)[0] == "chunked"


def test_invalid_arguments():
    assert fasa.select_layout(0, 10)[0] == "none"
    assert fasa.select_layout(10, 0)[0] == "none"
    assert fasa.select_layout(-5, -5)[0] == "none"


@pytest.mark.parametrize("n,budget,want", [
    (512, 64, ("whole", 512, 4, 0)),                # tiny fp32 case
    (32768, 256, ("chunked", 512, 4, 4096)),        # 32k layer: 2048 candidates
    (8192, 256, ("whole", 512, 16, 0)),             # ragged 4k-8k batch (longest row)
    (32768, 6193, ("whole_wide", 1024, 32, 0)),     # B = 6193, first step
    (32831, 6193, ("whole_wide", 1024, 40, 0)),     # B = 6193, last of 64 steps
    (131136, 1024, ("chunked", 1024, 16, 16384)),   # 128k workload's capacity
])
def test_workload_layouts(n, budget, want):
    assert fasa.select_layout(n, budget) == want


def test_decode_layout_filters_long_rows_with_fused_budgets():
    """A decode step selects through TIP's group maxima exactly when B <= 1024
    and 8192 < n <= 163840 (at most 10240 groups of 16, 20 per thread of 512);
    otherwise it uses the top-B layout fasa_select_layout reports."""
    # The 32k Llama-3-shaped layer and the 128k workload.
    assert fasa.decode_layout(32768, 256) == ("group_filter", 512, 4, 16)
    assert fasa.decode_layout(131072 + 31, 1024) == ("group_filter", 512, 20, 16)
    for n, budget in [(8192, 256), (32768, 1025), (163841, 16), (8193, 0), (6000, 100),
                      (200000, 1024)]:
        assert fasa.decode_layout(n, budget) == fasa.select_layout(n, budget), (n, budget)
    for n in (8193, 9000, 20000, 32768, 32769, 65536, 131103, 163840):
        for budget in (1, 256, 1024):
            kind, threads, per, chunk = fasa.decode_layout(n, budget)
            assert (kind, threads, chunk) == ("group_filter", 512, 16), (n, budget)
            assert per == (4 if -(-n // 16) <= 2048 else 20)
            assert threads * per >= -(-n // 16)
