"""Host-side accounting of the benchmark (no GPU): the split of row bytes
between the single-pass kernel and the binary32 cut-row kernel, and the
kernel names read from rocprofv3 traces."""
import numpy as np

import bench
from token_sampling_amd import workloads as W


def test_row_bytes_split_binary32_ragged():
    # 6 sessions of ragged in binary32: greedy sessions' target rows take the
    # single-pass kernel (top-k class); rule-2 sessions (T 0.8, top-p 0.95,
    # top-k off) take the cut-row kernel, target and draft rows
    w = W.make("ragged", sessions=6, logits="fp32")
    m = w.m.numpy().astype(np.int64)
    rule = w.rule.numpy()
    row = w.V * 4
    greedy = rule == 1
    stream = int((m[greedy] + 1).sum()) * row
    cut = int(((m + 1) + m)[~greedy].sum()) * row
    split = w.row_bytes_by_kernel()
    assert split == {"stream": stream, "dense32": cut}
    # together: every row a session's rule reads, once
    assert split["stream"] + split["dense32"] == \
        (int((m + 1).sum()) + int((m * (rule == 2)).sum())) * row
    # with published q rows no draft row is profiled
    q = w.row_bytes_by_kernel(q_rows=True)
    assert q["dense32"] == int((m + 1)[~greedy].sum()) * row


def test_row_bytes_split_bf16_is_all_single_pass():
    w = W.make("ragged", sessions=4)
    split = w.row_bytes_by_kernel()
    assert split["dense32"] == 0
    m = w.m.numpy().astype(np.int64)
    rule = w.rule.numpy()
    assert split["stream"] == (int((m + 1).sum()) + int((m * (rule == 2)).sum())) * w.V * 2


def test_kernel_short_names():
    names = {
        "void sv::(anonymous namespace)::k_rows_stream<sv::F32>(sv::F32::elem_t const*, int)":
            "k_rows_stream",
        "sv::(anonymous namespace)::k_rows_dense32(unsigned int const*, unsigned int const*)":
            "k_rows_dense32",
        "void sv::(anonymous namespace)::k_rows_split<4>(unsigned short const*)": "k_rows_split<4>",
        "void sv::(anonymous namespace)::k_finalize<sv::Bf16, false>(unsigned short const*)":
            "k_finalize",
        "void at::native::vectorized_elementwise_kernel<4, at::native::neg_kernel>()": "",
    }
    for full, short in names.items():
        assert bench.kernel_short_name(full) == short
