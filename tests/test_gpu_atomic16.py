"""bf16 dQ accumulation (dq_acc_dtype="bf16", the "atomic16" accumulation of "[ROCm] Fix
THD/ragged dQ backward on the bf16 dq_shuffle path (gfx950)"): packed bf16 atomic adds into a
bf16 accumulator with one slot per (segment, head), then scale and round into dq.

Tolerance.  dK and dV do not go through the accumulator, so they are held to the usual bar and
must equal the fp32 atomic mode's bit for bit (same arithmetic).  dQ adds one rounding to bf16
(unit roundoff u = 2^-8) per key tile's contribution and per running sum, so with n key tiles
per query row its relative rms error grows like u*sqrt(n/6) for contributions of similar size.
The cases here keep n <= 16 (<= 2048 keys), where the usual bar (cosine >= 0.9999, max|err| <=
2e-2 max|ref|) still holds with margin; one case at n = 32 checks the growth against the
looser bound u*sqrt(n)."""

import json
import os

import numpy as np
import pytest

from gpu_common import (assert_grads_close, make_inputs, metrics, oracle_backward, oracle_forward,
                        run_gpu, seq_offsets)

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
NONE, TL, BR, WIN = 0, 1, 2, 3

CASES = [
    # id, batch shape or segment lengths, heads, dims, mask, window
    ("batch_causal_d128", dict(B=2, Sq=1024, Sk=1024), (4, 4), (128, 128), TL, (-1, -1)),
    ("ragged_fixed_splits_a", dict(lens=[100, 80, 76]), (4, 2), (128, 128), TL, (-1, -1)),
    ("ragged_fixed_splits_b", dict(lens=[200, 56]), (4, 2), (128, 128), TL, (-1, -1)),
    ("ragged_window_gqa", dict(lens=[700, 130, 1000]), (8, 2), (128, 128), WIN, (150, 0)),
    ("batch_cross_d64_none", dict(B=2, Sq=200, Sk=900), (2, 2), (64, 64), NONE, (-1, -1)),
    ("batch_cross_d192_none", dict(B=1, Sq=130, Sk=700), (2, 1), (192, 128), NONE, (-1, -1)),
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
        x = make_inputs(seed, B=shape["B"], Sq=shape["Sq"], Sk=shape["Sk"], Hq=hq, Hkv=hkv,
                        d_qk=dqk, d_v=dv)
    return x, sq, sk, 1.0 / np.sqrt(dqk), mask, window


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_bf16_accumulator_matches_oracle(case):
    x, sq, sk, scale, mask, window = _inputs(case, 8101)
    o, lse = oracle_forward(x, scale=scale, mask=mask, window=window, sq=sq, sk=sk)
    ref = oracle_backward(x, scale=scale, mask=mask, window=window, sq=sq, sk=sk)
    got = run_gpu(x, o, lse, scale=scale, mask=mask, window=window, sq=sq, sk=sk,
                  deterministic=False, dq_acc_dtype="bf16")
    assert_grads_close(got, ref, sq, sk)


def test_bf16_accumulator_mixed_8192_packing():
    """The mixed 8192-token packing (fixed splits first, then seeded lengths) of the
    Llama-3-8B-shaped GQA workload, causal per segment, checked per segment: the layout class
    in which ragged segments after the first were lost."""
    lens = json.load(open(os.path.join(GOLDEN, "segments.json")))["mixed_8192"]
    sq = seq_offsets(lens)
    x = make_inputs(8102, lens_q=lens, lens_k=lens, Hq=32, Hkv=8, d_qk=128, d_v=128)
    o, lse = oracle_forward(x, scale=1 / np.sqrt(128), mask=TL, sq=sq, sk=sq)
    ref = oracle_backward(x, scale=1 / np.sqrt(128), mask=TL, sq=sq, sk=sq)
    got = run_gpu(x, o, lse, scale=1 / np.sqrt(128), mask=TL, sq=sq, sk=sq, deterministic=False,
                  dq_acc_dtype="bf16")
    assert_grads_close(got, ref, sq, sq)


def test_dk_dv_identical_across_accumulation_modes():
    """dK and dV never touch the dQ accumulator: all three modes give the same bits."""
    case = ("", dict(lens=[700, 130, 1000]), (8, 2), (128, 128), TL, (-1, -1))
    x, sq, sk, scale, mask, window = _inputs(case, 8103)
    o, lse = oracle_forward(x, scale=scale, mask=mask, sq=sq, sk=sk)
    runs = [run_gpu(x, o, lse, scale=scale, mask=mask, sq=sq, sk=sk, deterministic=det,
                    dq_acc_dtype=acc)
            for det, acc in ((True, "fp32"), (False, "fp32"), (False, "bf16"))]
    for other in runs[1:]:
        assert np.array_equal(runs[0][1], other[1])
        assert np.array_equal(runs[0][2], other[2])


def test_bf16_accumulator_error_growth_32_tiles():
    """4096 keys (32 key tiles per query row), no mask: dQ's relative rms error stays within
    u*sqrt(32), u = 2^-8, and well above the fp32 modes' error (the accumulation is really in
    bf16)."""
    x = make_inputs(8104, B=1, Sq=256, Sk=4096, Hq=2, Hkv=2, d_qk=128, d_v=128)
    scale = 1 / np.sqrt(128)
    o, lse = oracle_forward(x, scale=scale, mask=NONE)
    ref = oracle_backward(x, scale=scale, mask=NONE)
    got16 = run_gpu(x, o, lse, scale=scale, mask=NONE, deterministic=False, dq_acc_dtype="bf16")
    got32 = run_gpu(x, o, lse, scale=scale, mask=NONE, deterministic=False)

    def rel_rms(g, r):
        return float(np.linalg.norm(g - r) / np.linalg.norm(r))

    e16, e32 = rel_rms(got16[0], ref[0]), rel_rms(got32[0], ref[0])
    assert e16 <= 2.0 ** -8 * np.sqrt(32), "bf16 dQ relative rms error %.4g" % e16
    assert e16 > e32, (e16, e32)
    err, mref, _ = metrics(got16[0], ref[0])
    assert err <= 2e-2 * mref
