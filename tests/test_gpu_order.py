"""The longest-first list of the wide main kernel's work groups for ragged batches: the D stage's
first work group writes it to the end of the workspace, and it must be a permutation of the
grid ranked by the work group's step count (most first, ties in grid order).

The step count is recomputed here for top-left causal segments with as many queries as keys:
key tile j (256 keys from 256 j) is seen by the rows from 256 j to the segment's end, i.e.
(L - 1) // 32 - 8 j + 1 query blocks of 32 rows, for each of the G query heads of the K/V head;
an item's tiles add up, its parts take contiguous shares of that sum, and a non-empty work group
counts 6 more for its prologue and epilogue.  Cases: 896 work groups (a 1024-key sort), 1456
(2048 keys) and 1100 segments (the segment offsets are then read from global memory)."""

import numpy as np
import pytest

from attention_backward_fmha_amd import inputs as I

pytestmark = pytest.mark.gpu


def _steps(w, lens, hkv, g, T, P):
    nbh = hkv * len(lens)
    ip = w // nbh
    item, part = divmod(ip, P)
    L = lens[(w - ip * nbh) // hkv]
    steps = 0
    for j in range(item * T, item * T + T):
        if j * 256 >= L:
            break
        steps += ((L - 1) // 32 - (j * 256) // 32 + 1) * g
    if steps == 0:
        return 0
    return steps * (part + 1) // P - steps * part // P + 6


def _run(lens, hq, hkv):
    import torch
    import attention_backward_fmha_amd as F
    sq = I.seqstart(lens)
    t = int(sq[-1])
    z = lambda *s: torch.zeros(s, dtype=torch.bfloat16, device="cuda")
    q, k, v, o, do = z(t, hq, 128), z(t, hkv, 128), z(t, hkv, 128), z(t, hq, 128), z(t, hq, 128)
    lse = torch.zeros((hq, t), dtype=torch.float32, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    cu = torch.from_numpy(sq).cuda()
    c = F.make_call(q, k, v, o, lse, do, dq, dk, dv, mask_type=1, deterministic=True,
                    cu_seqlens_q=cu, cu_seqlens_k=cu, cu_seqlens_q_host=sq, cu_seqlens_k_host=sq,
                    tune=dict(kernel=F.KERNEL_WIDE))
    info = c.plan()
    n = info.ordered_groups
    ws = torch.full((c.workspace_size(),), 0xAB, dtype=torch.uint8, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    c.prepare(ws, s)
    c.run(ws, s)
    torch.cuda.synchronize()
    off = (info.dkv_acc_offset + info.dkv_acc_bytes + 255) // 256 * 256
    order = ws[off:off + 4 * n].cpu().numpy().view(np.int32)
    return info, n, order


CASES = [
    ("c3_packing", [1673, 226, 413, 527, 417, 1652, 1788, 1496], 32, 8, 896),
    ("mixed_packing", [100, 80, 76, 200, 56, 1673, 226, 413, 527, 417, 1652, 1788, 984], 32, 8, 1456),
    ("many_segments", [int(x) for x in np.random.default_rng(5).integers(1, 257, 1100)], 1, 1, 1100),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_work_group_order_is_a_ranked_permutation(case):
    _, lens, hq, hkv, expect_n = case
    info, n, order = _run(lens, hq, hkv)
    assert n == expect_n
    assert np.array_equal(np.sort(order), np.arange(n))
    cost = [_steps(int(w), lens, hkv, hq // hkv, info.tiles_per_item, info.kv_parts) for w in order]
    keys = [(-c, int(w)) for c, w in zip(cost, order)]
    assert all(a < b for a, b in zip(keys, keys[1:]))
    assert cost[0] > 0


def test_keys_without_queries_still_get_their_list():
    """Every query segment empty: the D stage has no rows, yet the main kernel's work groups
    still take their items from the list, so the ranking work group runs on its own. The
    workspace starts zeroed (a stale list whose entries are all in range, which would run item 0
    everywhere) and dK/dV start as NaN: every key must come back with dK = dV = 0."""
    import torch
    import attention_backward_fmha_amd as F
    lens_q, lens_k = [0, 0, 0], [300, 700, 50]
    sq, sk = I.seqstart(lens_q), I.seqstart(lens_k)
    tk = int(sk[-1])
    g = torch.Generator(device="cpu").manual_seed(11)
    kv = lambda: torch.randn((tk, 2, 128), generator=g).to(torch.bfloat16).cuda()
    z = lambda *s: torch.zeros(s, dtype=torch.bfloat16, device="cuda")
    q, o, do = z(0, 4, 128), z(0, 4, 128), z(0, 4, 128)
    k, v = kv(), kv()
    lse = torch.zeros((4, 0), dtype=torch.float32, device="cuda")
    dq = torch.empty_like(q)
    dk = torch.full_like(k, float("nan"))
    dv = torch.full_like(v, float("nan"))
    c = F.make_call(q, k, v, o, lse, do, dq, dk, dv, mask_type=0, deterministic=True,
                    cu_seqlens_q=torch.from_numpy(sq).cuda(), cu_seqlens_k=torch.from_numpy(sk).cuda(),
                    cu_seqlens_q_host=sq, cu_seqlens_k_host=sk, tune=dict(kernel=F.KERNEL_WIDE))
    info = c.plan()
    n = info.ordered_groups
    assert info.rows_q == 0 and n > 1
    ws = torch.zeros(c.workspace_size(), dtype=torch.uint8, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    c.prepare(ws, s)
    c.run(ws, s)
    torch.cuda.synchronize()
    off = (info.dkv_acc_offset + info.dkv_acc_bytes + 255) // 256 * 256
    order = ws[off:off + 4 * n].cpu().numpy().view(np.int32)
    assert np.array_equal(np.sort(order), np.arange(n))
    assert torch.equal(dk.float().cpu(), torch.zeros(dk.shape))
    assert torch.equal(dv.float().cpu(), torch.zeros(dv.shape))
