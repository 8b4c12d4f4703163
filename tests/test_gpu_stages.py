"""GPU tests of single stages, determinism and degenerate shapes, through the C ABI."""

import numpy as np
import pytest

import oracle
from attention_backward_fmha_amd import inputs as I
from gpu_common import assert_grads_close, make_inputs, oracle_backward, oracle_forward, seq_offsets

pytestmark = pytest.mark.gpu

NONE, TL, BR, WIN = 0, 1, 2, 3


def _setup(x, o, lse, *, scale, mask, window=(-1, -1), sq=None, sk=None, deterministic=True):
    import torch
    import attention_backward_fmha_amd as F
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16).cuda()
    q, k, v, do = (dev(x[n]) for n in ("q", "k", "v", "do"))
    od = dev(I.round_bf16(o.astype(np.float32)))
    ld = torch.from_numpy(lse.astype(np.float32)).cuda()
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    kw = {}
    if sq is not None:
        kw = dict(cu_seqlens_q=torch.from_numpy(sq).cuda(), cu_seqlens_k=torch.from_numpy(sk).cuda(),
                  cu_seqlens_q_host=sq, cu_seqlens_k_host=sk)
    call = F.make_call(q, k, v, od, ld, do, dq, dk, dv, scale=scale, mask_type=mask, window=window,
                       deterministic=deterministic, **kw)
    ws = torch.empty(call.workspace_size(), dtype=torch.uint8, device="cuda")
    return call, ws, (q, k, v, od, ld, do, dq, dk, dv)


def test_dot_stage_matches_rowsum():
    import torch
    import attention_backward_fmha_amd as F
    lens = [100, 80, 76]
    sq = seq_offsets(lens)
    x = make_inputs(4001, lens_q=lens, lens_k=lens, Hq=8, Hkv=2, d_qk=128, d_v=128)
    o, lse = oracle_forward(x, scale=0.088, mask=TL, sq=sq, sk=sq)
    call, ws, t = _setup(x, o, lse, scale=0.088, mask=TL, sq=sq, sk=sq)
    stream = torch.cuda.current_stream().cuda_stream
    call.prepare(ws, stream)
    call.run(ws, stream, F.STAGE_DOT)
    torch.cuda.synchronize()
    info = call.plan()
    d = ws[info.d_offset:info.d_offset + 4 * 8 * info.rows_q].view(torch.float32).view(8, -1).cpu().numpy()
    ob = t[3].float().cpu().numpy()
    ref = oracle.rowsum_product(x["do"], ob).T  # [Hq, rows]
    np.testing.assert_allclose(d, ref, rtol=1e-5, atol=1e-5 * np.abs(ref).max())


def _touch(mask, window, lq, lk, tm, tn):
    """(q-block, key-tile) pairs with at least one allowed (row, key) pair, by brute force."""
    ok = oracle.allowed(mask, window[0], window[1], lq, lk)
    nb, nt = -(-lq // tm), -(-lk // tn)
    return {(i, j) for i in range(nb) for j in range(nt)
            if ok[i * tm:(i + 1) * tm, j * tn:(j + 1) * tn].any()}


def _block_offsets(tm, d):
    """Offset of element (r, c) inside a deterministic accumulator block, as documented with
    fmha_bwd_plan_info: 32x32 tiles t = (r/32)*(d/32) + c/32 at 1024*t, element (r, c) of a
    tile at 256*(r/8) + 4*(c + 32*((r/4)%2)) + r%4."""
    r = np.arange(tm)[:, None]
    c = np.arange(d)[None, :]
    t = (r // 32) * (d // 32) + c // 32
    rr, cc = r % 32, c % 32
    return 1024 * t + 256 * (rr // 8) + 4 * (cc + 32 * ((rr // 4) % 2)) + rr % 4


@pytest.mark.parametrize("mask,window", [(NONE, (-1, -1)), (TL, (-1, -1)), (WIN, (100, 0))])
def test_reduce_stage_is_bit_exact(mask, window):
    """Partials placed in the accumulator by hand; untouched splits and the padding rows past
    each segment hold NaN, so reading one would show.  Expected bits from the oracle's
    ascending fp32 split sum and RNE rounding."""
    import torch
    import attention_backward_fmha_amd as F
    lens = [300, 77, 512]
    sq = seq_offsets(lens)
    hq, d = 4, 128
    x = make_inputs(4002, lens_q=lens, lens_k=lens, Hq=hq, Hkv=2, d_qk=d, d_v=d)
    o = np.zeros((sum(lens), hq, d))
    lse = np.zeros((hq, sum(lens)))
    call, ws, t = _setup(x, o, lse, scale=0.125, mask=mask, window=window, sq=sq, sk=sq)
    info = call.plan()
    rows = info.rows_q
    tm, tn = info.tile_m, info.tile_n
    assert info.acc_rows == rows + len(lens) * tm
    acc = ws[info.dq_acc_offset:info.dq_acc_offset + info.dq_acc_bytes].view(torch.float32)
    rng = np.random.default_rng(9)
    parts = (rng.standard_normal((info.nsplits, hq, rows, d)) * 10).astype(np.float32)
    dev = np.full((info.nsplits, hq, info.acc_rows * d), np.nan, np.float32)
    offs = _block_offsets(tm, d)
    expect = np.zeros((rows, hq, d), np.uint16)
    for b in range(len(lens)):
        r0 = int(sq[b])
        touched = _touch(mask, window, lens[b], lens[b], tm, tn)
        for i in range(-(-lens[b] // tm)):
            nr = min(lens[b], (i + 1) * tm) - i * tm
            rs = slice(r0 + i * tm, r0 + i * tm + nr)
            # split s holds key tiles s*T .. s*T + T - 1 (T = tiles_per_item)
            used = sorted({j // info.tiles_per_item for (ii, j) in touched if ii == i})
            base = (r0 + b * tm + i * tm) * d
            for j in used:
                dev[j, :, base + offs[:nr].ravel()] = parts[j, :, rs, :].reshape(hq, -1).T
            sel = parts[used][:, :, rs, :] if used else np.zeros((0, hq, nr, d), np.float32)
            expect[rs] = oracle.dq_split_reduce(sel, 0.125).transpose(1, 0, 2)
    acc.copy_(torch.from_numpy(dev.ravel()))
    stream = torch.cuda.current_stream().cuda_stream
    call.run(ws, stream, F.STAGE_REDUCE)
    torch.cuda.synchronize()
    got = t[6].view(torch.int16).cpu().numpy().view(np.uint16)
    np.testing.assert_array_equal(got, expect)


def test_reduce_stage_atomic_mode_is_bit_exact():
    import torch
    import attention_backward_fmha_amd as F
    x = make_inputs(4003, B=2, Sq=100, Sk=70, Hq=2, Hkv=2, d_qk=64, d_v=64)
    call, ws, t = _setup(x, np.zeros((2, 100, 2, 64)), np.zeros((2, 2, 100)), scale=0.3, mask=BR,
                         deterministic=False)
    info = call.plan()
    assert info.nsplits == 1
    parts = (np.random.default_rng(3).standard_normal((1, 2, 200, 64)) * 5).astype(np.float32)
    acc = ws[info.dq_acc_offset:info.dq_acc_offset + info.dq_acc_bytes].view(torch.float32)
    acc.copy_(torch.from_numpy(parts.ravel()))
    call.run(ws, torch.cuda.current_stream().cuda_stream, F.STAGE_REDUCE)
    torch.cuda.synchronize()
    got = t[6].view(torch.int16).cpu().numpy().view(np.uint16)  # [B, Sq, H, d]
    exp = oracle.dq_split_reduce(parts, 0.3)  # [H, B*Sq, d]
    np.testing.assert_array_equal(got, exp.reshape(2, 2, 100, 64).transpose(1, 2, 0, 3))


def test_prepare_zeroes_the_atomic_accumulator():
    import torch
    x = make_inputs(4004, B=1, Sq=64, Sk=64, Hq=1, Hkv=1, d_qk=64, d_v=64)
    call, ws, _ = _setup(x, np.zeros((1, 64, 1, 64)), np.zeros((1, 1, 64)), scale=0.1, mask=NONE,
                         deterministic=False)
    info = call.plan()
    ws.fill_(0x7F)
    call.prepare(ws, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    acc = ws[info.dq_acc_offset:info.dq_acc_offset + info.dq_acc_bytes]
    assert int(acc.count_nonzero()) == 0


@pytest.mark.parametrize("d", [128, 64, 192], ids=["d128", "d64_128rows", "d192"])
def test_deterministic_mode_is_bit_identical_over_10_runs(d):
    import torch
    import attention_backward_fmha_amd as F
    lens = [700, 130, 1000]
    sq = seq_offsets(lens)
    x = make_inputs(4005, lens_q=lens, lens_k=lens, Hq=8, Hkv=2, d_qk=d, d_v=min(d, 128))
    o, lse = oracle_forward(x, scale=0.088, mask=TL, sq=sq, sk=sq)
    call, ws, t = _setup(x, o, lse, scale=0.088, mask=TL, sq=sq, sk=sq)
    stream = torch.cuda.current_stream().cuda_stream
    outs = []
    for _ in range(10):
        ws.fill_(0xFF)  # stale workspace contents must not matter
        for g in t[6:]:
            g.fill_(1.0)
        call.prepare(ws, stream)
        call.run(ws, stream)
        torch.cuda.synchronize()
        outs.append([g.view(torch.int16).cpu().numpy().copy() for g in t[6:]])
    for run in outs[1:]:
        for a, b in zip(outs[0], run):
            np.testing.assert_array_equal(a, b)
    ref = oracle_backward(x, scale=0.088, mask=TL, sq=sq, sk=sq)
    got = tuple(g.float().cpu().numpy().astype(np.float64) for g in t[6:])
    assert_grads_close(got, ref, sq=sq, sk=sq)


@pytest.mark.parametrize("Sq,Sk", [(0, 100), (100, 0), (1, 1), (1, 300), (300, 1)])
@pytest.mark.parametrize("deterministic", [True, False], ids=["det", "atomic"])
def test_degenerate_lengths(Sq, Sk, deterministic):
    import torch
    import attention_backward_fmha_amd as F
    x = make_inputs(4006, B=2, Sq=Sq, Sk=Sk, Hq=2, Hkv=1, d_qk=64, d_v=64)
    o, lse = oracle_forward(x, scale=0.125, mask=NONE)
    ref = oracle_backward(x, scale=0.125, mask=NONE)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16).cuda()
    dq, dk, dv = F.bwd(dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(I.round_bf16(o.astype(np.float32))),
                       torch.from_numpy(lse.astype(np.float32)).cuda(), dev(x["do"]), scale=0.125,
                       deterministic=deterministic)
    torch.cuda.synchronize()
    got = tuple(g.float().cpu().numpy().astype(np.float64) for g in (dq, dk, dv))
    for g, r in zip(got, ref):
        assert g.shape == r.shape
        if r.size:
            assert np.all(np.isfinite(g))
            if np.abs(r).max() == 0.0:
                # exactly zero in exact arithmetic (one key: dS = P (dP - D) = 0); the kernel's D
                # uses the bf16-rounded O, so only rounding-level residue may remain
                assert np.abs(g).max() <= 1e-4
            else:
                np.testing.assert_allclose(g, r, atol=2e-2 * np.abs(r).max())


def test_noncontiguous_strides():
    """Q/K/V/dO as views into wider buffers (head-interleaved QKV-style packing)."""
    import torch
    import attention_backward_fmha_amd as F
    B, S, H, d = 2, 150, 4, 128
    x = make_inputs(4007, B=B, Sq=S, Sk=S, Hq=H, Hkv=H, d_qk=d, d_v=d)
    o, lse = oracle_forward(x, scale=0.088, mask=TL)
    ref = oracle_backward(x, scale=0.088, mask=TL)
    packed = torch.zeros((B, S, 3, H, d), dtype=torch.bfloat16, device="cuda")
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16).cuda()
    packed[:, :, 0] = dev(x["q"])
    packed[:, :, 1] = dev(x["k"])
    packed[:, :, 2] = dev(x["v"])
    lse_wide = torch.zeros((B, H, S + 10), dtype=torch.float32, device="cuda")
    lse_wide[:, :, :S] = torch.from_numpy(lse.astype(np.float32)).cuda()
    dq, dk, dv = F.bwd(packed[:, :, 0], packed[:, :, 1], packed[:, :, 2],
                       dev(I.round_bf16(o.astype(np.float32))), lse_wide[:, :, :S], dev(x["do"]),
                       scale=0.088, mask_type=TL)
    torch.cuda.synchronize()
    got = tuple(g.float().cpu().numpy().astype(np.float64) for g in (dq, dk, dv))
    assert_grads_close(got, ref)
