"""Padded THD: each segment sits at the start of a longer slot of physical rows (cu_seqlens next
to cu_seqlens_padded, the layout of "[ROCm] Fix THD/ragged dQ backward on the bf16 dq_shuffle
path (gfx950)").  The slot tails of every input hold NaN, so reading one would show; the slot
tails of dq/dk/dv hold a sentinel that must survive.  Reference: the oracle on the compact
(unpadded) segments."""

import numpy as np
import pytest

from attention_backward_fmha_amd import inputs as I
from gpu_common import assert_grads_close, make_inputs, oracle_backward, oracle_forward, seq_offsets

pytestmark = pytest.mark.gpu

SENTINEL = 0x7F01  # a bf16 NaN bit pattern no kernel writes


def _scatter(compact, starts, slots, lens, fill):
    """Rows of each segment at the start of its slot; the tails get `fill`."""
    out = np.full((int(slots[-1]),) + compact.shape[1:], fill, compact.dtype)
    for b, n in enumerate(lens):
        out[slots[b]:slots[b] + n] = compact[starts[b]:starts[b] + n]
    return out


def _run(lens_q, lens_k, slots_q, slots_k, *, mask, hq, hkv, d, deterministic, seed, dq_acc_dtype="fp32"):
    import torch
    import attention_backward_fmha_amd as F
    sq, sk = seq_offsets(lens_q), seq_offsets(lens_k)
    pq, pk = np.asarray(slots_q, np.int32), np.asarray(slots_k, np.int32)
    x = make_inputs(seed, lens_q=lens_q, lens_k=lens_k, Hq=hq, Hkv=hkv, d_qk=d, d_v=d)
    scale = 1.0 / np.sqrt(d)
    o, lse = oracle_forward(x, scale=scale, mask=mask, sq=sq, sk=sk)
    ref = oracle_backward(x, scale=scale, mask=mask, sq=sq, sk=sk)

    def dev_bf16(a, starts, slots, lens):
        return torch.from_numpy(_scatter(np.asarray(a, np.float32), starts, slots, lens, np.nan)).to(
            torch.bfloat16).cuda()

    q = dev_bf16(x["q"], sq, pq, lens_q)
    k = dev_bf16(x["k"], sk, pk, lens_k)
    v = dev_bf16(x["v"], sk, pk, lens_k)
    do = dev_bf16(x["do"], sq, pq, lens_q)
    od = dev_bf16(I.round_bf16(o.astype(np.float32)), sq, pq, lens_q)
    ld = torch.from_numpy(np.ascontiguousarray(
        _scatter(lse.T.astype(np.float32), sq, pq, lens_q, np.nan).T)).cuda()  # [Hq, T_phys]
    outs = []
    for t in (q, k, v):
        o_ = torch.empty_like(t)
        o_.view(torch.int16).fill_(SENTINEL - 0x10000 if SENTINEL >= 0x8000 else SENTINEL)
        outs.append(o_)
    dq, dk, dv = F.bwd(q, k, v, od, ld, do, scale=scale, mask_type=mask, deterministic=deterministic,
                       cu_seqlens_q=torch.from_numpy(sq).cuda(), cu_seqlens_k=torch.from_numpy(sk).cuda(),
                       cu_seqlens_q_host=sq, cu_seqlens_k_host=sk,
                       cu_seqlens_q_padded=torch.from_numpy(pq).cuda(),
                       cu_seqlens_k_padded=torch.from_numpy(pk).cuda(),
                       cu_seqlens_q_padded_host=pq, cu_seqlens_k_padded_host=pk, out=tuple(outs),
                       dq_acc_dtype=dq_acc_dtype)
    torch.cuda.synchronize()
    bits = [t.view(torch.int16).cpu().numpy().view(np.uint16) for t in (dq, dk, dv)]
    got = [t.float().cpu().numpy().astype(np.float64) for t in (dq, dk, dv)]
    # slot tails untouched; segment rows gathered back into the compact layout
    compact = []
    for g, bt, starts, slots, lens in ((got[0], bits[0], sq, pq, lens_q), (got[1], bits[1], sk, pk, lens_k),
                                       (got[2], bits[2], sk, pk, lens_k)):
        rows = np.concatenate([np.arange(slots[b], slots[b] + n) for b, n in enumerate(lens)] + [[]]).astype(int)
        tail = np.setdiff1d(np.arange(int(slots[-1])), rows)
        assert np.all(bt[tail] == SENTINEL), "a padding row was written"
        compact.append(g[rows])
    assert_grads_close(compact, ref, sq, sk)


@pytest.mark.parametrize("deterministic", [True, False], ids=["det", "atomic"])
def test_padded_thd_pad16_causal(deterministic):
    """Segments of 103, 77 and 61 tokens, each padded to a multiple of 16 (241 -> 256 rows)."""
    lens = [103, 77, 61]
    slots = [0, 112, 192, 256]
    _run(lens, lens, slots, slots, mask=1, hq=4, hkv=2, d=128, deterministic=deterministic, seed=5101)


@pytest.mark.parametrize("deterministic", [True, False], ids=["det", "atomic"])
def test_padded_thd_long_slots_gqa(deterministic):
    """[100, 80, 76] in 192-row slots (tails longer than a query block), GQA 8/2, causal."""
    lens = [100, 80, 76]
    slots = [0, 192, 384, 576]
    _run(lens, lens, slots, slots, mask=1, hq=8, hkv=2, d=128, deterministic=deterministic, seed=5102)


def test_padded_thd_cross_lengths_no_mask():
    """Different q and k lengths and slots, one empty segment, d=64, no mask."""
    lens_q, lens_k = [50, 0, 30], [70, 5, 20]
    slots_q, slots_k = [0, 64, 80, 144], [0, 80, 96, 128]
    _run(lens_q, lens_k, slots_q, slots_k, mask=0, hq=2, hkv=1, d=64, deterministic=True, seed=5103)


def test_padded_thd_pad16_causal_bf16_accumulator():
    """The bf16 (atomic16) accumulator on the padded layout of the pages' fix: 103/77/61 tokens
    in 112/80/64-row slots; its slots are indexed by logical position, so the tensors' padding
    cannot move them."""
    lens = [103, 77, 61]
    slots = [0, 112, 192, 256]
    _run(lens, lens, slots, slots, mask=1, hq=4, hkv=2, d=128, deterministic=False, seed=5101,
         dq_acc_dtype="bf16")
