"""fmha_bwd_run_noalloc, the entry point for callers that cannot allocate device memory: its
results (computed in the library's static scratch) against fmha_bwd_prepare_workspace +
fmha_bwd_run with a caller-allocated workspace on the same inputs, on two calls in a row, the
second with a smaller input, in the deterministic (bit-identical) and fp32-atomic modes, and
against the oracle at the target's bar."""

import ctypes
import sys

import numpy as np
import pytest

from attention_backward_fmha_amd import _lib
from gpu_common import (assert_close, assert_grads_close, make_inputs, oracle_backward,
                        oracle_forward, seq_offsets, to_dev_bf16, to_dev_f32)

pytestmark = pytest.mark.gpu

TL = 1  # causal, top-left


def _device_case(x, o, lse, sq):
    import torch
    dev = {n: to_dev_bf16(x[n]) for n in ("q", "k", "v", "do")}
    from attention_backward_fmha_amd import inputs as I
    dev["o"] = to_dev_bf16(I.round_bf16(o.astype(np.float32)))
    dev["lse"] = to_dev_f32(lse.astype(np.float32))
    seq = {}
    if sq is not None:
        sq32 = np.asarray(sq, np.int32)
        seq = dict(cu_seqlens_q=torch.from_numpy(sq32).cuda(), cu_seqlens_k=torch.from_numpy(sq32).cuda(),
                   cu_seqlens_q_host=sq32, cu_seqlens_k_host=sq32)
    return dev, seq


def _run_both(dev, seq, scale, deterministic):
    """(prepare + run with a torch workspace, run_noalloc) outputs as float64 arrays."""
    import torch
    import attention_backward_fmha_amd as F
    outs = []
    for noalloc in (False, True):
        dq = torch.full_like(dev["q"], float("nan"))
        dk = torch.full_like(dev["k"], float("nan"))
        dv = torch.full_like(dev["v"], float("nan"))
        call = F.make_call(dev["q"], dev["k"], dev["v"], dev["o"], dev["lse"], dev["do"], dq, dk, dv,
                           scale=scale, mask_type=TL, deterministic=deterministic, **seq)
        stream = torch.cuda.current_stream().cuda_stream
        if noalloc:
            assert call.workspace_size() <= _lib.NOALLOC_MAX_BYTES
            call.run_noalloc(stream)
        else:
            ws = torch.empty(call.workspace_size(), dtype=torch.uint8, device="cuda")
            call.prepare(ws, stream)
            call.run(ws, stream)
        torch.cuda.synchronize()
        outs.append(tuple(t.float().cpu().numpy().astype(np.float64) for t in (dq, dk, dv)))
    return outs


CASES = [
    # first call: batch mode, GQA, 1000 rows (several key tiles and a ragged tail)
    dict(name="bshd_2x8x1000_gqa", seed=9301, B=2, S=1000, Hq=8, Hkv=2, lens=None),
    # second call, smaller: ragged segments, lengths not multiples of 16
    dict(name="thd_300_77_129", seed=9302, B=None, S=None, Hq=4, Hkv=2, lens=[300, 77, 129]),
]


def test_noalloc_matches_caller_workspace_on_two_calls():
    scale = 1.0 / np.sqrt(128)
    for case in CASES:
        if case["lens"] is None:
            x = make_inputs(case["seed"], B=case["B"], Sq=case["S"], Sk=case["S"], Hq=case["Hq"],
                            Hkv=case["Hkv"], d_qk=128, d_v=128)
            sq = None
        else:
            sq = seq_offsets(case["lens"])
            x = make_inputs(case["seed"], lens_q=case["lens"], lens_k=case["lens"], Hq=case["Hq"],
                            Hkv=case["Hkv"], d_qk=128, d_v=128)
        o, lse = oracle_forward(x, scale=scale, mask=TL, sq=sq, sk=sq)
        ref = oracle_backward(x, scale=scale, mask=TL, sq=sq, sk=sq)
        dev, seq = _device_case(x, o, lse, sq)
        for det in (True, False):
            print("case %s deterministic=%s" % (case["name"], det), file=sys.stderr, flush=True)
            base, got = _run_both(dev, seq, scale, det)
            for n, g, b in zip(("dq", "dk", "dv"), got, base):
                assert np.all(np.isfinite(g)), n
                if det or n != "dq":  # same kernels and order: the same bits
                    assert np.array_equal(g, b), "%s %s differs from the caller-workspace run" % (case["name"], n)
                else:  # fp32 atomics: the order of the adds may differ
                    assert_close("%s %s vs caller workspace" % (case["name"], n), g, b)
            assert_grads_close(got, ref, sq, sq, label="%s det=%s: " % (case["name"], det))


def test_noalloc_rejects_a_workspace_beyond_its_scratch():
    import torch
    import attention_backward_fmha_amd as F
    # deterministic 2x16x2048 causal needs about 270 MB of splits: more than the scratch
    q = torch.zeros((2, 2048, 16, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros((2, 16, 2048), dtype=torch.float32, device="cuda")
    call = F.make_call(q, q, q, q, lse, q, q, q, q, mask_type=TL, deterministic=True)
    assert call.workspace_size() > _lib.NOALLOC_MAX_BYTES
    st = _lib.lib().fmha_bwd_run_noalloc(ctypes.byref(call.args), None)
    assert st == _lib.ERR_WORKSPACE_TOO_SMALL
