"""The workspace header: prepare writes a magic value and the plan fingerprint; with
FMHA_BWD_DEBUG=1 a run whose arguments plan a different layout than the prepared one fails
with FMHA_ERR_PLAN_MISMATCH instead of reading a workspace laid out for other segments (the
sizing/run disagreement of "[ROCm] Fix THD/ragged dQ backward on the bf16 dq_shuffle path
(gfx950)", Root cause)."""

import numpy as np
import pytest

from attention_backward_fmha_amd import inputs as I

pytestmark = pytest.mark.gpu


def _call(lens, mask, deterministic=True):
    import torch
    import attention_backward_fmha_amd as F
    sq = I.seqstart(lens)
    t = int(sq[-1])
    dev = lambda *s: torch.zeros(s, dtype=torch.bfloat16, device="cuda")
    q, k, v, o, do = dev(t, 4, 128), dev(t, 2, 128), dev(t, 2, 128), dev(t, 4, 128), dev(t, 4, 128)
    lse = torch.zeros((4, t), dtype=torch.float32, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    cu = torch.from_numpy(sq).cuda()
    return F.make_call(q, k, v, o, lse, do, dq, dk, dv, mask_type=mask, deterministic=deterministic,
                       cu_seqlens_q=cu, cu_seqlens_k=cu, cu_seqlens_q_host=sq, cu_seqlens_k_host=sq)


def test_matching_arguments_pass_the_debug_check(monkeypatch):
    import torch
    monkeypatch.setenv("FMHA_BWD_DEBUG", "1")
    for det in (True, False):
        c = _call([100, 80, 76], 1, det)
        ws = torch.empty(c.workspace_size(), dtype=torch.uint8, device="cuda")
        s = torch.cuda.current_stream().cuda_stream
        c.prepare(ws, s)
        c.run(ws, s)
        torch.cuda.synchronize()


def test_other_arguments_are_a_plan_mismatch(monkeypatch):
    import torch
    from attention_backward_fmha_amd import _lib
    monkeypatch.setenv("FMHA_BWD_DEBUG", "1")
    s = torch.cuda.current_stream().cuda_stream
    a = _call([100, 80, 76], 1)
    for b in (_call([100, 80, 76], 0),      # another mask, same sizes
              _call([80, 100, 76], 1)):     # the same tokens segmented differently
        n = max(a.workspace_size(), b.workspace_size())
        ws = torch.empty(n, dtype=torch.uint8, device="cuda")
        a.prepare(ws, s)
        with pytest.raises(_lib.FmhaError) as e:
            b.run(ws, s)
        assert e.value.status == _lib.ERR_PLAN_MISMATCH
    # a workspace that was never prepared
    ws = torch.zeros(a.workspace_size(), dtype=torch.uint8, device="cuda")
    with pytest.raises(_lib.FmhaError) as e:
        a.run(ws, s)
    assert e.value.status == _lib.ERR_PLAN_MISMATCH
    torch.cuda.synchronize()


def test_without_debug_the_header_is_not_read(monkeypatch):
    import torch
    monkeypatch.delenv("FMHA_BWD_DEBUG", raising=False)
    a = _call([100, 80, 76], 1)
    ws = torch.zeros(a.workspace_size(), dtype=torch.uint8, device="cuda")
    a.run(ws, torch.cuda.current_stream().cuda_stream)  # deterministic mode needs no zeroing
    torch.cuda.synchronize()
