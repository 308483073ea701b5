"""The counter summaries under profiles/ must describe the kernels as they are.

bench.py reports counted HBM traffic and matrix-unit work only while the
sources a kernel is built from hash to the value recorded beside its
counters.  These CPU checks fail as soon as a kernel source changes without
the rocprofv3 passes being taken again, so a stale profile cannot go
unnoticed."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402

KERNELS = ["prepare_kernel<bf16,false>", "scan_split_kernel<false>", "scan_head_kernel<false>",
           "scan_head_kernel<true>", "decode_step_kernel@B64", "attn_fwd_kernel",
           "attn_decode_kernel", "bwd_chain_split_kernel", "bwd_grad_kernel"]


@pytest.mark.parametrize("kernel", KERNELS)
def test_traffic_line_matches_sources(kernel):
    assert bench.counted_traffic(kernel) is not None, (
        "profiles/hbm_bytes_bench_workloads.md has no line for %s keyed to the current "
        "sources: take the FETCH_SIZE / WRITE_SIZE passes again" % kernel)


def test_mfma_line_matches_sources():
    assert bench.counted_mfma_gflop() is not None, (
        "profiles/mfma_ops_bench_workloads.md is not keyed to the current prefill sources")
