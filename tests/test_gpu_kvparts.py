"""Key tiles whose steps (query heads x query blocks) are split over several work groups
(tune_kv_parts forces the count; the plan uses parts when there are too few K/V heads and
tiles to fill the GPU), in both main-kernel layouts at d = 128.  Each part adds fp32 dK/dV partials and a final pass sums them in
ascending part order, so deterministic mode stays bit-reproducible."""

import numpy as np
import pytest

import attention_backward_fmha_amd as F

from gpu_common import assert_grads_close, make_inputs, oracle_backward, oracle_forward, run_gpu, seq_offsets

pytestmark = pytest.mark.gpu
NONE, TL, BR, WIN = 0, 1, 2, 3

CASES = [
    ("ragged_causal_gqa", dict(lens=[300, 77, 512]), (8, 2), (128, 128), TL, (-1, -1)),
    ("batch_window_d64", dict(B=2, Sq=257, Sk=257), (4, 2), (64, 64), WIN, (40, 3)),
    ("batch3_causal_d128", dict(B=3, Sq=200, Sk=200), (2, 1), (128, 128), BR, (-1, -1)),
    ("batch_cross_d192", dict(B=1, Sq=130, Sk=333), (4, 1), (192, 128), NONE, (-1, -1)),
    ("batch_br_lq_gt_lk", dict(B=1, Sq=300, Sk=90), (2, 2), (128, 128), BR, (-1, -1)),
]


def _inputs(case, seed):
    _, shape, (hq, hkv), (dqk, dv), mask, window = case
    if "lens" in shape:
        lens = shape["lens"]
        sq = sk = seq_offsets(lens)
        x = make_inputs(seed, lens_q=lens, lens_k=lens, Hq=hq, Hkv=hkv, d_qk=dqk, d_v=dv)
    else:
        sq = sk = None
        x = make_inputs(seed, B=shape["B"], Sq=shape["Sq"], Sk=shape["Sk"], Hq=hq, Hkv=hkv, d_qk=dqk, d_v=dv)
    return x, sq, sk, 1.0 / np.sqrt(dqk), mask, window


# (case, kernel): both layouts where d = 128 or 64 selects the wide one by default
CASE_KERNELS = [(c, k) for c in CASES for k in ([F.KERNEL_AUTO, F.KERNEL_FOUR_WAVE] if c[3] in ((128, 128), (64, 64))
                                                 else [F.KERNEL_AUTO])]
CK_IDS = ["%s-%s" % (c[0], {F.KERNEL_AUTO: "auto", F.KERNEL_FOUR_WAVE: "four_wave"}[k]) for c, k in CASE_KERNELS]


@pytest.mark.parametrize("mode", ["det", "atomic", "atomic16"])
@pytest.mark.parametrize("parts", [1, 3, 8])
@pytest.mark.parametrize("case,kernel", CASE_KERNELS, ids=CK_IDS)
def test_split_key_tiles_match_oracle(case, kernel, parts, mode):
    tune = dict(kv_parts=parts, kernel=kernel)
    x, sq, sk, scale, mask, window = _inputs(case, 9401)
    o, lse = oracle_forward(x, scale=scale, mask=mask, window=window, sq=sq, sk=sk)
    ref = oracle_backward(x, scale=scale, mask=mask, window=window, sq=sq, sk=sk)
    det, acc = {"det": (True, "fp32"), "atomic": (False, "fp32"), "atomic16": (False, "bf16")}[mode]
    got = run_gpu(x, o, lse, scale=scale, mask=mask, window=window, sq=sq, sk=sk, deterministic=det,
                  dq_acc_dtype=acc, tune=tune)
    assert_grads_close(got, ref, sq, sk)


@pytest.mark.parametrize("tiles", [2, 4, 8])
@pytest.mark.parametrize("parts", [3, 8])
@pytest.mark.parametrize("case,kernel", CASE_KERNELS, ids=CK_IDS)
def test_parts_of_multi_tile_items_match_oracle(case, kernel, parts, tiles):
    """Deterministic items of several key tiles, split into parts: a part adds its dQ partial
    of a later tile onto the split blocks it wrote for an earlier one."""
    tune = dict(kv_parts=parts, tiles_per_item=tiles, kernel=kernel)
    x, sq, sk, scale, mask, window = _inputs(case, 9403)
    o, lse = oracle_forward(x, scale=scale, mask=mask, window=window, sq=sq, sk=sk)
    ref = oracle_backward(x, scale=scale, mask=mask, window=window, sq=sq, sk=sk)
    got = run_gpu(x, o, lse, scale=scale, mask=mask, window=window, sq=sq, sk=sk, tune=tune)
    assert_grads_close(got, ref, sq, sk)


@pytest.mark.parametrize("kernel", [F.KERNEL_WIDE, F.KERNEL_FOUR_WAVE], ids=["wide", "four_wave"])
@pytest.mark.parametrize("tiles", [1, 2])
def test_split_key_tiles_are_bit_identical(tiles, kernel):
    tune = dict(kv_parts=5, tiles_per_item=tiles, kernel=kernel)
    x, sq, sk, scale, mask, window = _inputs(CASES[0], 9402)
    o, lse = oracle_forward(x, scale=scale, mask=mask, sq=sq, sk=sk)
    first = run_gpu(x, o, lse, scale=scale, mask=mask, sq=sq, sk=sk, tune=tune)
    for _ in range(4):
        again = run_gpu(x, o, lse, scale=scale, mask=mask, sq=sq, sk=sk, tune=tune)
        for a, b in zip(first, again):
            assert np.array_equal(a, b)
