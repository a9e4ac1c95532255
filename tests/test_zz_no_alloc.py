"""ssd_forward_fused_static (the fused forward on the library's static scratch
array, for callers that cannot allocate) against ssd_forward(SSD_ALGO_FUSED)
with a caller workspace: the same kernels, so the same bits.  Two calls in a
row, the second on a smaller problem (the array keeps the first call's
contents), a packed batch, and the size limit."""
import numpy as np
import pytest
import torch

from mamba_ssd_chunked_scan_amd import ssd
from helpers import device_inputs, make_inputs, small_workload, with_initial_states

pytestmark = pytest.mark.gpu


def both(w, out_dtype=torch.float32):
    inp = with_initial_states(make_inputs(w))
    dev = device_inputs(inp, torch.bfloat16)
    args = (dev["x"], dev["B"], dev["C"], dev["dt"], dev["A"], dev["dt_bias"], dev["D"],
            dev["z"], dev["initial_states"])
    ref = ssd.ssd_forward(*args, cu_seqlens=dev["cu_seqlens"], chunk_size=128, algo="fused",
                          out_dtype=out_dtype)
    out = torch.full(dev["x"].shape, float("nan"), dtype=out_dtype, device="cuda")
    fin = torch.full(dev["initial_states"].shape, float("nan"), dtype=torch.float32,
                     device="cuda")
    got = ssd.ssd_forward_fused_static(*args, cu_seqlens=dev["cu_seqlens"], out=out,
                                       final_states=fin)
    torch.cuda.synchronize()
    return ref, got


def test_static_scratch_matches_workspace_path_twice_shrinking():
    big = small_workload("big", seqlen=8192, nheads=64, headdim=64, ngroups=8, dstate=128,
                         chunk_size=128)
    small = small_workload("small", seqlen=777, nheads=8, headdim=64, ngroups=2, dstate=64,
                           chunk_size=128, seed=8)
    for w in (big, small):
        ref, got = both(w)
        assert torch.equal(got[0], ref[0]) and torch.equal(got[1], ref[1]), w.name


def test_static_scratch_packed_and_bf16_out():
    w = small_workload("packed", seqlen=3000, nheads=16, headdim=64, ngroups=4, dstate=128,
                       chunk_size=128, seqlens=(1000, 0, 1, 1999))
    ref, got = both(w, out_dtype=torch.bfloat16)
    assert torch.equal(got[0], ref[0]) and torch.equal(got[1], ref[1])


def test_static_scratch_rejects_a_problem_beyond_the_array():
    # 2048 heads x 64 rows: 2048 units of 32 KiB aggregates = 64 MiB > 32 MiB
    x = torch.zeros((1, 256, 2048, 64), dtype=torch.bfloat16, device="cuda")
    B = torch.zeros((1, 256, 1, 128), dtype=torch.bfloat16, device="cuda")
    dt = torch.zeros((1, 256, 2048), dtype=torch.bfloat16, device="cuda")
    A = -torch.ones(2048, dtype=torch.float32, device="cuda")
    prob = ssd.problem_from(x, B, 128)
    assert prob.workspace_size("fused") > (32 << 20)
    with pytest.raises(ssd.SSDError) as e:
        ssd.ssd_forward_fused_static(x, B, B, dt, A)
    assert e.value.status == 6
    assert "static" in str(e.value)
