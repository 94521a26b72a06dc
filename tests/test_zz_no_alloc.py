"""The entry point that allocates nothing (sv_verify_noalloc), through the C
ABI: its outputs equal sv_verify's (same inputs, its own workspace) bit for
bit, on two calls in a row, the second with a smaller input; sizes beyond its
array are refused before anything is enqueued."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from tests import parity
from tests.test_gpu_parity import mixed_case
from token_sampling_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def svm():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import token_sampling_amd as sv
    sv.lib()
    return sv


def noalloc_call(sv, t, d, tokens, m, rule, smp, seed, round_, probe=True):
    B, M1, V = t.shape
    M = M1 - 1
    dev = t.device
    out = {"accepted_len": torch.full((B,), -7, dtype=torch.int32, device=dev),
           "out_tokens": torch.full((B, M + 1), -7, dtype=torch.int32, device=dev)}
    pr = None
    if probe:
        out["p_tok"] = torch.full((B, M), -7.0, dtype=torch.float64, device=dev)
        out["q_tok"] = torch.full((B, M), -7.0, dtype=torch.float64, device=dev)
        pr = ctypes.byref(sv._Probe(out["p_tok"].data_ptr(), out["q_tok"].data_ptr()))
    dt = sv.BF16 if t.dtype == torch.bfloat16 else sv.FP32
    rc = sv.lib().sv_verify_noalloc(
        t.data_ptr(), None if d is None else d.data_ptr(), dt, tokens.data_ptr(), m.data_ptr(),
        rule.data_ptr(), smp.data_ptr(), B, M, V, seed, round_, out["accepted_len"].data_ptr(),
        out["out_tokens"].data_ptr(), pr, torch.cuda.current_stream(dev).cuda_stream)
    assert rc == sv.OK, sv.strerror(rc)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


def same(a, b):
    for k in a:
        assert np.array_equal(a[k], b[k]), k


def test_noalloc_matches_sv_verify_twice_second_smaller(svm):
    sv = svm
    # first call: the B=256, M=8, V=128256 workload (top-k 50, top-p 0.9)
    parity.log("[case] no-alloc entry: b256 workload, then a smaller mixed batch")
    w = W.make("b256_topk_topp", device="cuda")
    smp = w.sampling_tensor("cuda")
    ref = {k: v.cpu().numpy() for k, v in
           sv.verify(w.target, w.draft, w.tokens, w.m, w.rule, smp, w.seed, w.round,
                     probe=True).items()}
    got = noalloc_call(sv, w.target, w.draft, w.tokens, w.m, w.rule, smp, w.seed, w.round)
    same(ref, got)
    assert (got["accepted_len"] >= 0).sum() > 200
    del w
    torch.cuda.empty_cache()
    # second call, smaller: mixed profiles (dense and top-k rows, greedy and
    # sampling, -inf masks), which also draw from whole rows
    h = mixed_case(71, 20, 5, 3000, "bf16")
    dev = "cuda"
    t, d = parity.to_device(h["target"]), parity.to_device(h["draft"])
    args = (parity.to_device(np.asarray(h["tokens"], np.int32)),
            parity.to_device(np.asarray(h["m"], np.int32)),
            parity.to_device(np.asarray(h["rule"], np.int32)),
            parity.sampling_bytes(h["sampling"], dev))
    ref2 = {k: v.cpu().numpy() for k, v in
            sv.verify(t, d, *args, h["seed"], h["round"], probe=True).items()}
    got2 = noalloc_call(sv, t, d, *args, h["seed"], h["round"])
    same(ref2, got2)
    # and the oracle agrees with both
    parity.compare(got2, parity.run_oracle(h), "noalloc-small")


def test_noalloc_refuses_sizes_beyond_its_array(svm):
    sv = svm
    B, M, V = 1 << 20, 8, 1 << 20
    assert sv.workspace_bytes(B, M, V) > (128 << 20)
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: the call returns first
    rc = sv.lib().sv_verify_noalloc(fake, fake, sv.BF16, fake, fake, fake, fake, B, M, V, 0, 1,
                                    fake, fake, None, None)
    assert rc == sv.ERR_WORKSPACE
    rc = sv.lib().sv_verify_noalloc(fake, fake, sv.BF16, fake, fake, fake, fake, 0, M, V, 0, 1,
                                    fake, fake, None, None)
    assert rc == sv.ERR_ARG
