"""Strided tensors: Q, K, V as views into one packed [.., Hq + 2*Hkv, d] buffer (the packed
QKV layout of fused-attention callers), dQ/dK/dV as views into a packed gradient buffer, O
and dO with a padded head stride, and LSE with a padded sequence stride.  Results must match
the oracle, and no byte of the packed output buffer outside the three views may change."""

import numpy as np
import pytest

from attention_backward_fmha_amd import inputs as I
from gpu_common import assert_grads_close, make_inputs, oracle_backward, oracle_forward, seq_offsets

pytestmark = pytest.mark.gpu
SENTINEL = 0x7F01  # a bf16 NaN pattern that no kernel writes


def _bf16(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16).cuda()


@pytest.mark.parametrize("mode", ["det", "atomic", "atomic16"])
@pytest.mark.parametrize("layout", ["bshd", "thd"])
def test_packed_qkv_views_and_padded_strides(layout, mode):
    import torch
    import attention_backward_fmha_amd as F
    hq, hkv, d = 8, 2, 128
    scale = 1 / np.sqrt(d)
    if layout == "bshd":
        B, S = 2, 300
        x = make_inputs(9301, B=B, Sq=S, Sk=S, Hq=hq, Hkv=hkv, d_qk=d, d_v=d)
        sq = sk = None
        lead = (B, S)
    else:
        lens = [100, 80, 76, 200, 56]
        sq = sk = seq_offsets(lens)
        x = make_inputs(9302, lens_q=lens, lens_k=lens, Hq=hq, Hkv=hkv, d_qk=d, d_v=d)
        lead = (int(sq[-1]),)
    o, lse = oracle_forward(x, scale=scale, mask=1, sq=sq, sk=sk)
    ref = oracle_backward(x, scale=scale, mask=1, sq=sq, sk=sk)

    nh = hq + 2 * hkv
    qkv = torch.empty(lead + (nh, d), dtype=torch.bfloat16, device="cuda")
    qkv[..., :hq, :] = _bf16(x["q"])
    qkv[..., hq:hq + hkv, :] = _bf16(x["k"])
    qkv[..., hq + hkv:, :] = _bf16(x["v"])
    q, k, v = qkv[..., :hq, :], qkv[..., hq:hq + hkv, :], qkv[..., hq + hkv:, :]
    # O and dO with one spare head of padding per row
    opad = torch.zeros(lead + (hq + 1, d), dtype=torch.bfloat16, device="cuda")
    opad[..., :hq, :] = _bf16(I.round_bf16(o.astype(np.float32)))
    dopad = torch.zeros(lead + (hq + 1, d), dtype=torch.bfloat16, device="cuda")
    dopad[..., :hq, :] = _bf16(x["do"])
    # LSE with 8 spare positions per row of the sequence axis
    if layout == "bshd":
        lpad = torch.zeros((lead[0], hq, lead[1] + 8), dtype=torch.float32, device="cuda")
        lpad[..., :lead[1]] = torch.from_numpy(lse.astype(np.float32)).cuda()
        lse_v = lpad[..., :lead[1]]
    else:
        lpad = torch.zeros((hq, lead[0] + 8), dtype=torch.float32, device="cuda")
        lpad[:, :lead[0]] = torch.from_numpy(lse.astype(np.float32)).cuda()
        lse_v = lpad[:, :lead[0]]
    dqkv = torch.empty(lead + (nh + 1, d), dtype=torch.bfloat16, device="cuda")
    dqkv.view(torch.int16).fill_(SENTINEL)
    out = (dqkv[..., :hq, :], dqkv[..., hq:hq + hkv, :], dqkv[..., hq + hkv:nh, :])
    kw = {}
    if sq is not None:
        kw = dict(cu_seqlens_q=torch.from_numpy(sq).cuda(), cu_seqlens_k=torch.from_numpy(sk).cuda(),
                  cu_seqlens_q_host=sq, cu_seqlens_k_host=sk)
    det, acc = {"det": (True, "fp32"), "atomic": (False, "fp32"), "atomic16": (False, "bf16")}[mode]
    F.bwd(q, k, v, opad[..., :hq, :], lse_v, dopad[..., :hq, :], scale=scale, mask_type=1,
          deterministic=det, dq_acc_dtype=acc, out=out, **kw)
    torch.cuda.synchronize()
    got = [t.float().cpu().numpy().astype(np.float64) for t in out]
    assert_grads_close(got, ref, sq, sk)
    spare = dqkv[..., nh:, :].view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.all(spare == SENTINEL), "a byte outside the dQ/dK/dV views was written"
