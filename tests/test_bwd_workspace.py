"""Workspace of the per-chunk backward (ssd_backward_ex_workspace_size, host
code only): the two fp32 state buffers that grow with the heads are taken in
head passes of at most 256 MiB by default (whole groups, or multiples of eight
heads of one group), so the full-size workloads stay near or below 350 MB."""
import pytest

from mamba_ssd_chunked_scan_amd import ssd

MB = 1e6


def size(T, H, P, G, N, C=128):
    return ssd.Problem(1, T, H, P, G, N, C).backward_workspace_size("fused")


def state_bytes(T, H, P, N):
    # the forward carry-in states and their gradients, fp32, 128-token chunks
    return 2 * -(-T // 128) * H * P * N * 4


@pytest.mark.parametrize("T,H,G,limit_mb", [
    (16384, 64, 8, 350),   # two Nemotron-Nano lengths: two passes of 32 heads (4 groups)
    (8192, 128, 1, 350),   # twice Granite's length: one group, two passes of 64 heads
    (65536, 80, 1, 400),   # long context: one group of 80 heads, passes of 8
])
def test_full_size_workloads_take_head_passes(T, H, G, limit_mb):
    full_states = state_bytes(T, H, 64, 128)
    got = size(T, H, 64, G, 128)
    assert got <= limit_mb * MB, f"{got / MB:.1f} MB"
    assert got < full_states          # fewer heads than the problem per pass
    assert got >= state_bytes(T, 8, 64, 128)   # at least one pass's states


@pytest.mark.parametrize("T,H,G", [(8192, 64, 8), (4096, 128, 1)])
def test_benchmark_workloads_take_one_pass(T, H, G):
    # Nemotron-Nano and Granite: the two state buffers of every head fit the
    # default pass budget of 256 MiB (Granite's one group of 128 heads adds
    # the dB/dC partials of its sixteen eight-head splits)
    got = size(T, H, 64, G, 128)
    assert state_bytes(T, H, 64, 128) <= got <= 350 * MB


def test_small_problems_take_one_pass():
    # everything fits: the size is the one-pass layout, and it grows with the heads
    a, b = size(1000, 8, 64, 4, 64), size(1000, 16, 64, 8, 64)
    assert state_bytes(1000, 8, 64, 64) < a < b


def test_passes_are_balanced():
    # 64 heads over two passes of 32 heads: the pass states are half the problem's
    T, H, N = 16384, 64, 128
    got = size(T, H, 64, 8, N)
    half = state_bytes(T, H // 2, 64, N)
    assert half <= got < half + 16 * MB
