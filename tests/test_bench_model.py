"""The benchmark's roofline denominators (algorithmic bytes and useful flops per
launch) against figures worked out by hand from the per-stage definitions: each
input read once, each output written once, causal halves only.

Real path, fp32 chunk states, bf16 inputs and outputs (MB = 1e6 bytes):
  Nemotron-Nano (T 8192, 64 x 64 heads, d_state 128, 8 groups, chunk 128):
    chunk cumsum 3.15, C.B^T 50.5, chunk state 220, state passing 271,
    chunk scan 371, fused forward 238 (x, B, C, dt, z, out, final states)
  Granite-style (T 4096, 128 x 64 heads, 1 group): chunk state 204, state
    passing 273, chunk scan 340, fused 209
  Long context (T 65536, 80 heads, chunk 256, no z): chunk state 1380, state
    passing 1345, chunk scan 2085, fused 1389
Complex path at the 434M shape (batch 8, T 2048, 16 x 64 heads, d_state 64,
chunk 64; complex64 = 8 bytes): x, B, C are 134.2 MB each, the chunk states
134.2 MB, the real output 67.1 MB, dt 1.0 MB:
  chunk state = x + B + dt + states + step sums = 403.7 MB, 8 K H C P N flops = 8.59 GF
  state passing = 2 states + step sums + final = 272.6 MB
  chunk scan = x + B + C + dt + states + out = 605.0 MB
"""
import pytest

import bench
from mamba_ssd_chunked_scan_amd.inputs import COMPLEX_WORKLOADS, WORKLOADS


def model(name):
    w = WORKLOADS[name]
    K = w.batch * (-(-w.seqlen // w.chunk_size))
    return bench.stage_bytes(w, K, 4, 2, 2), bench.stage_flops(w, K)


@pytest.mark.parametrize("name,expect", [
    ("nemotron", {"chunk_cumsum": 3.15, "bmm_chunk": 50.5, "chunk_state": 220,
                  "state_passing": 271, "chunk_scan": 371, "fused_fwd": 238}),
    ("granite", {"chunk_state": 204, "state_passing": 273, "chunk_scan": 340, "fused_fwd": 209}),
    ("longctx", {"chunk_state": 1380, "state_passing": 1345, "chunk_scan": 2085,
                 "fused_fwd": 1389}),
])
def test_real_path_bytes(name, expect):
    nb, _ = model(name)
    for k, mb in expect.items():
        assert abs(nb[k] / 1e6 - mb) <= 0.01 * mb, (k, nb[k] / 1e6, mb)


def test_real_path_flops_nemotron():
    _, nf = model("nemotron")
    # chunk state: 2 K H C P N = 2 * 64 * 64 * 128 * 64 * 128
    assert nf["chunk_state"] == 2 * 64 * 64 * 128 * 64 * 128
    # fused forward: C.B^T (causal) + chunk state + chunk scan (causal), 22.6 GF
    assert abs(nf["fused_fwd"] / 1e9 - 22.6) < 0.05


def test_complex_model():
    nb, nf = bench.complex_stage_model(COMPLEX_WORKLOADS["complex_434m"])
    expect = {"cx_chunk_state": 403.7, "cx_state_passing": 272.6, "cx_chunk_scan": 605.0}
    for k, mb in expect.items():
        assert abs(nb[k] / 1e6 - mb) <= 0.001 * mb, (k, nb[k] / 1e6, mb)
    assert abs(nf["cx_chunk_state"] / 1e9 - 8.59) < 0.01
