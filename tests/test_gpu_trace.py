"""The profiling hook fpr_trace_set, which bench.py's per-stage times and live
roofline read, and whose launch order rocprof_summary.py uses to attribute a
kernel trace's launches to stages: every launch of a step gets its stage
name, in launch order, with its own pair of events on the launch stream;
`only` keeps one stage; a full trace stops recording instead of writing past
its capacity."""
import pytest
import torch

import gpu_run
from fp8_packed_reduced_amd import binding as B
from fp8_packed_reduced_amd import inputs
from fp8_packed_reduced_amd import rocprof_summary as R

pytestmark = pytest.mark.gpu

TINY = inputs.WORKLOADS["tiny"]
assert TINY["d_qk"] in (64, 96, 128), "the fused forward's stage order"


def _traced(fn, capacity=64, only=None):
    tr = B.KernelTrace(capacity, only=only)
    with tr:
        fn()
    torch.cuda.synchronize()
    return tr.records()


@pytest.mark.parametrize("pack_forward", [True, False])
def test_trace_names_every_launch_of_a_qkv_step(pack_forward):
    recs = _traced(lambda: gpu_run.run(TINY, pack_forward=pack_forward))
    names = [n for n, _ in recs]
    assert names == R.step_order("step_64k", separate_pack=not pack_forward)
    assert all(ms > 0.0 for _, ms in recs)


@pytest.mark.parametrize("pack_forward", [True, False])
def test_trace_names_every_launch_of_an_mlp_step(pack_forward):
    recs = _traced(lambda: gpu_run.run_mlp(inputs.MLP_WORKLOADS["mlp_tiny"],
                                           pack_forward=pack_forward))
    names = [n for n, _ in recs]
    assert names == R.step_order("mlp_64k", separate_pack=not pack_forward)
    assert all(ms > 0.0 for _, ms in recs)


def test_trace_only_keeps_one_stage():
    recs = _traced(lambda: gpu_run.run(TINY, pack_forward=True), only="gemm_fwd")
    assert [n for n, _ in recs] == ["gemm_fwd"]


def test_trace_stops_at_capacity():
    full = R.step_order("step_64k")
    recs = _traced(lambda: gpu_run.run(TINY, pack_forward=True), capacity=3)
    assert [n for n, _ in recs] == full[:3]


def test_trace_ends_with_its_context():
    tr = B.KernelTrace(64)
    with tr:
        gpu_run.run(TINY, pack_forward=True)
    torch.cuda.synchronize()
    n = len(tr.records())
    assert n == len(R.step_order("step_64k"))
    gpu_run.run(TINY, pack_forward=True)  # tracing is off: nothing more recorded
    torch.cuda.synchronize()
    assert len(tr.records()) == n
