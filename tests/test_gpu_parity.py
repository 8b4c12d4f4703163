"""GPU parity of the HIP path against the fp64 oracle, element by element, at sizes the oracle
finishes in seconds that still span several tiles and ragged tails."""

import json
import os

import numpy as np
import pytest

import attention_backward_fmha_amd as F
from gpu_common import (assert_grads_close, make_inputs, oracle_backward, oracle_forward,
                        run_gpu, seq_offsets)

pytestmark = pytest.mark.gpu

NONE, TL, BR, WIN = 0, 1, 2, 3
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _segments():
    with open(os.path.join(GOLDEN, "segments.json")) as f:
        return json.load(f)


# main-kernel layouts at d = 128 and 64: the default (eight waves, 256-key tiles) and the
# four-wave one
KERNELS = [F.KERNEL_AUTO, F.KERNEL_FOUR_WAVE]
KERNEL_IDS = ["wide", "four_wave"]


def _run_batch(seed, B, Sq, Sk, Hq, Hkv, d_qk, d_v, mask, window=(-1, -1), deterministic=True,
               sigmas=(1, 1, 1, 1), kernel=F.KERNEL_AUTO):
    x = make_inputs(seed, B=B, Sq=Sq, Sk=Sk, Hq=Hq, Hkv=Hkv, d_qk=d_qk, d_v=d_v, sigmas=sigmas)
    scale = 1.0 / np.sqrt(d_qk)
    o, lse = oracle_forward(x, scale=scale, mask=mask, window=window)
    ref = oracle_backward(x, scale=scale, mask=mask, window=window)
    got = run_gpu(x, o, lse, scale=scale, mask=mask, window=window, deterministic=deterministic,
                  tune=dict(kernel=kernel))
    assert_grads_close(got, ref)


def _run_group(seed, lens_q, lens_k, Hq, Hkv, d_qk, d_v, mask, window=(-1, -1), deterministic=True,
               kernel=F.KERNEL_AUTO):
    sq, sk = seq_offsets(lens_q), seq_offsets(lens_k)
    x = make_inputs(seed, lens_q=lens_q, lens_k=lens_k, Hq=Hq, Hkv=Hkv, d_qk=d_qk, d_v=d_v)
    scale = 1.0 / np.sqrt(d_qk)
    o, lse = oracle_forward(x, scale=scale, mask=mask, window=window, sq=sq, sk=sk)
    ref = oracle_backward(x, scale=scale, mask=mask, window=window, sq=sq, sk=sk)
    got = run_gpu(x, o, lse, scale=scale, mask=mask, window=window, sq=sq, sk=sk,
                  deterministic=deterministic, tune=dict(kernel=kernel))
    assert_grads_close(got, ref, sq=sq, sk=sk)


def test_tiny_no_mask_d64():
    """B=1, H=1, S=64, d=64, no mask, deterministic; fp32 N(0,1) draws rounded to bf16."""
    _run_batch(1001, 1, 64, 64, 1, 1, 64, 64, NONE)


@pytest.mark.parametrize("kernel", KERNELS, ids=KERNEL_IDS)
@pytest.mark.parametrize("deterministic", [True, False], ids=["det", "atomic"])
@pytest.mark.parametrize("mask,window", [(NONE, (-1, -1)), (TL, (-1, -1)), (BR, (-1, -1)),
                                         (WIN, (37, 5)), (WIN, (-1, 20)), (WIN, (70, -1))],
                         ids=["none", "tl", "br", "win37_5", "win_l_inf", "win_r_inf"])
def test_batch_masks_d128(mask, window, deterministic, kernel):
    # Sq != Sk and neither a multiple of the tiles: several tiles plus ragged tails
    _run_batch(2001, 2, 200, 333, 4, 2, 128, 128, mask, window, deterministic, kernel=kernel)


@pytest.mark.parametrize("d_qk,d_v,kernel", [(64, 64, F.KERNEL_AUTO), (64, 64, F.KERNEL_FOUR_WAVE),
                                             (192, 128, F.KERNEL_AUTO)],
                         ids=["d64_wide", "d64_four_wave", "d192"])
@pytest.mark.parametrize("mask", [NONE, BR])
def test_batch_head_dims(d_qk, d_v, kernel, mask):
    _run_batch(2002, 2, 150, 290, 2, 1, d_qk, d_v, mask, sigmas=(1, 1, 0.5, 0.5), kernel=kernel)


@pytest.mark.parametrize("name", ["split_100_80_76", "split_200_56", "split_103_77_61",
                                  "split_64x4", "split_128_128", "single_256"])
@pytest.mark.parametrize("kernel", KERNELS, ids=KERNEL_IDS)
@pytest.mark.parametrize("deterministic", [True, False], ids=["det", "atomic"])
def test_group_fixed_packings_causal(name, deterministic, kernel):
    lens = _segments()["fixed_from_pages"][name]
    _run_group(3001, lens, lens, 8, 2, 128, 128, TL, deterministic=deterministic, kernel=kernel)


def test_group_empty_and_uneven_segments():
    lens_q = [70, 0, 129, 1, 64]
    lens_k = [33, 12, 200, 0, 64]
    for mask in (NONE, TL, BR):
        _run_group(3002, lens_q, lens_k, 4, 4, 128, 128, mask)


def test_bottom_right_rows_without_keys():
    # Lq > Lk with bottom-right causal: the first Lq - Lk rows see no key (dQ = 0)
    _run_batch(2003, 1, 300, 100, 2, 2, 64, 64, BR)


@pytest.mark.parametrize("kernel", KERNELS, ids=KERNEL_IDS)
@pytest.mark.parametrize("mode", ["det", "atomic", "atomic16"])
@pytest.mark.parametrize("mask,window", [(TL, (-1, -1)), (BR, (-1, -1)), (WIN, (90, 7)), (NONE, (-1, -1))],
                         ids=["tl", "br", "win90_7", "none"])
def test_group_d64_block_heights(mask, window, mode, kernel):
    """d = 64 in both layouts: the wide one (32-row query blocks, the default) and the four-wave
    one, which takes 128-row blocks in the deterministic and bf16-accumulator modes and 64-row
    blocks with fp32 atomics: ragged segments around 32/64/128-row boundaries (2, 63..65,
    127..129, 255, 300 queries), GQA 6/2, every mode.  Every segment has rows with two or more
    allowed keys under each mask (where no row does, the exact dQ is 0 and a relative bar cannot
    hold)."""
    lens_q = [2, 63, 64, 65, 127, 128, 129, 255, 300]
    lens_k = [7, 65, 64, 200, 128, 3, 129, 255, 290]
    sq, sk = seq_offsets(lens_q), seq_offsets(lens_k)
    x = make_inputs(3101, lens_q=lens_q, lens_k=lens_k, Hq=6, Hkv=2, d_qk=64, d_v=64)
    scale = 1.0 / np.sqrt(64)
    o, lse = oracle_forward(x, scale=scale, mask=mask, window=window, sq=sq, sk=sk)
    ref = oracle_backward(x, scale=scale, mask=mask, window=window, sq=sq, sk=sk)
    det, acc = {"det": (True, "fp32"), "atomic": (False, "fp32"), "atomic16": (False, "bf16")}[mode]
    got = run_gpu(x, o, lse, scale=scale, mask=mask, window=window, sq=sq, sk=sk,
                  deterministic=det, dq_acc_dtype=acc, tune=dict(kernel=kernel))
    assert_grads_close(got, ref, sq=sq, sk=sk)
