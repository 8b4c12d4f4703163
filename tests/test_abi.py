"""CPU tests of the C ABI: the library loads and exports every declared entry point, and the
host-only entry points (workspace sizing, plan query) validate arguments and agree with each
other.  No compute call is made (there may be no GPU here)."""

import ctypes
import json
import os
import re
import subprocess

import numpy as np
import pytest

from attention_backward_fmha_amd import _lib
from attention_backward_fmha_amd._lib import Args

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fmha_bwd.h")
GOLDEN = os.path.join(ROOT, "tests", "golden")
FAKE = 1 << 20  # a 16-byte aligned non-null address (never dereferenced by host entry points)


@pytest.fixture(scope="session", autouse=True)
def built_library():
    if not os.path.exists(_lib.LIB_PATH):
        from attention_backward_fmha_amd import build
        build.build()
    return _lib.lib()


def declared_functions():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"FMHA_BWD_API\s+[\w\s\*]+?\b(fmha_(?:bwd|fwd)_\w+)\s*\(", src)))


def test_header_declarations_are_exported():
    names = declared_functions()
    assert set(names) == set(_lib.EXPORTS)
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if ln.strip()}
    for n in names:
        assert n in exported, n
    # nothing but the C ABI leaks out of the library
    ours = {e for e in exported if "fmha" in e}
    assert ours == set(names)


def test_struct_layout_matches_header():
    """Offsets of the ctypes mirror against a C compile of the header."""
    src = """
#include <stddef.h>
#include <stdio.h>
#include "fmha_bwd.h"
#define F(m) printf("\\"%s\\": %zu,\\n", #m, offsetof(fmha_bwd_args, m));
#define G(m) printf("\\"%s\\": %zu,\\n", #m, offsetof(fmha_bwd_plan_info, m));
int main(void) {
  printf("{\\n");
  F(B) F(scale) F(deterministic) F(seqstart_q_host) F(seqstart_k_dev) F(q) F(lse) F(dv)
  F(q_stride) F(dv_stride) F(lse_stride) F(seqstart_q_padded_host) F(seqstart_k_padded_dev)
  F(dq_acc_dtype) F(bias) F(dbias_stride) F(bias_h) F(p_drop) F(philox_seed) F(philox_offset)
  G(nsplits) G(rows_q) G(workspace_bytes) G(flops) G(acc_rows) G(dq_acc_elem_bytes) G(dbias_acc_bytes)
  G(reduce_read_bytes) G(kv_parts) G(dkv_acc_bytes)
  printf("\\"size_args\\": %zu, \\"size_info\\": %zu}\\n", sizeof(fmha_bwd_args), sizeof(fmha_bwd_plan_info));
  return 0;
}
"""
    import tempfile
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "t.c")
        exe = os.path.join(d, "t")
        open(c, "w").write(src)
        subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), c, "-o", exe], check=True)
        ref = json.loads(subprocess.run([exe], capture_output=True, text=True, check=True).stdout)
    assert ref["size_args"] == ctypes.sizeof(Args)
    assert ref["size_info"] == ctypes.sizeof(_lib.PlanInfo)
    for k, v in ref.items():
        if k.startswith("size"):
            continue
        cls = _lib.PlanInfo if k in ("nsplits", "rows_q", "workspace_bytes", "flops", "acc_rows",
                                     "dq_acc_elem_bytes", "dbias_acc_bytes", "reduce_read_bytes",
                                     "kv_parts", "dkv_acc_bytes") else Args
        assert getattr(cls, k).offset == v, k


def test_mask_numbering_matches_pages():
    """Mask numbering from the mask-type table of the TransformerEngine PR 446 review."""
    table = json.load(open(os.path.join(GOLDEN, "mask_encoding.json")))
    src = open(HEADER).read()
    for name, value in table["numbering"].items():
        assert re.search(r"\b%s\s*=\s*%d\b" % (name, value), src), name
        assert getattr(_lib, name.replace("FMHA_", "")) == value


def batch_args(B=2, Hq=4, Hkv=2, Sq=200, Sk=333, d_qk=128, d_v=128, mask=0, window=(-1, -1),
               deterministic=1, kernel=_lib.KERNEL_FOUR_WAVE):
    """Arguments with fake device pointers.  The layout rules most tests here check are the
    four-wave kernel's, so that kernel is requested unless `kernel` says otherwise."""
    a = Args(B=B, Hq=Hq, Hkv=Hkv, Sq=Sq, Sk=Sk, d_qk=d_qk, d_v=d_v, scale=1.0 / np.sqrt(d_qk),
             mask_type=mask, window_left=window[0], window_right=window[1],
             deterministic=deterministic, tune_kernel=kernel)
    for n in ("q", "k", "v", "o", "dout", "lse", "dq", "dk", "dv"):
        setattr(a, n, FAKE)
    for n, H, d, S in (("q_stride", Hq, d_qk, Sq), ("k_stride", Hkv, d_qk, Sk), ("v_stride", Hkv, d_v, Sk),
                       ("o_stride", Hq, d_v, Sq), ("do_stride", Hq, d_v, Sq), ("dq_stride", Hq, d_qk, Sq),
                       ("dk_stride", Hkv, d_qk, Sk), ("dv_stride", Hkv, d_v, Sk)):
        arr = getattr(a, n)
        arr[0], arr[1], arr[2] = S * H * d, H * d, d
    a.lse_stride[0] = Hq * Sq
    a.lse_stride[1] = Sq
    return a


def group_args(lens_q, lens_k, Hq=4, Hkv=2, d=128, mask=1, deterministic=1,
               kernel=_lib.KERNEL_FOUR_WAVE):
    sq = np.concatenate([[0], np.cumsum(lens_q)]).astype(np.int32)
    sk = np.concatenate([[0], np.cumsum(lens_k)]).astype(np.int32)
    a = batch_args(B=len(lens_q), Hq=Hq, Hkv=Hkv, Sq=max(lens_q), Sk=max(lens_k), d_qk=d, d_v=d,
                   mask=mask, deterministic=deterministic, kernel=kernel)
    a.seqstart_q_host = sq.ctypes.data
    a.seqstart_k_host = sk.ctypes.data
    a.seqstart_q_dev = FAKE
    a.seqstart_k_dev = FAKE
    a._keep = (sq, sk)
    return a


def status_of(a):
    n = ctypes.c_size_t(0)
    return _lib.lib().fmha_bwd_workspace_size(ctypes.byref(a), ctypes.byref(n))


def test_workspace_size_and_plan_agree():
    for det in (0, 1):
        a = batch_args(deterministic=det)
        info = _lib.plan_query(a)
        assert _lib.workspace_size(a) == info.workspace_bytes
        rows = 2 * 200
        assert info.rows_q == rows
        # ceil(333 / 128) = 3 key tiles; 6 work items at most, so one tile per item
        assert info.tiles_per_item == 1
        assert info.nsplits == (3 if det else 1)
        assert info.needs_zero == (0 if det else 1)
        # deterministic blocks get tile_m rows of padding per segment
        assert info.acc_rows == rows + (2 * info.tile_m if det else 0)
        assert info.dq_acc_bytes == info.nsplits * 4 * info.acc_rows * 128 * 4
        assert info.dq_acc_offset % 256 == 0 and info.workspace_bytes % 256 == 0
        assert info.dq_acc_offset + info.dq_acc_bytes <= info.workspace_bytes
        # nsplits never exceeds ceil(max Sk / 16)
        assert info.nsplits <= -(-333 // 16)


def test_workspace_starts_with_its_header():
    """Bytes 0..255 hold the header prepare writes; D follows, then L, the accumulator."""
    info = _lib.plan_query(batch_args())
    assert info.d_offset == 256
    assert info.dq_acc_offset >= 256 + 2 * 4 * 2 * 200 * 4  # D and L: [Hq][rows] fp32 each
    assert _lib.status_string(_lib.ERR_PLAN_MISMATCH) == "FMHA_ERR_PLAN_MISMATCH"


def test_group_mode_uses_physical_rows():
    lens = [100, 80, 76]
    a = group_args(lens, lens)
    info = _lib.plan_query(a)
    assert info.group_mode == 1
    assert info.rows_q == 256
    assert info.nsplits == 1  # longest segment has 100 keys: one 128-key tile
    # empty segments are fine and contribute no rows
    b = group_args([5, 0, 7], [0, 3, 9])
    assert _lib.plan_query(b).rows_q == 12


def test_forward_argument_errors():
    """fmha_fwd_run checks its arguments before any device work: o and lse are required, the
    backward-only tensors are not (a missing one is no error, so the call reaches the launch,
    which needs a GPU and is not made here)."""
    L = _lib.lib()
    a = batch_args()
    a.o = None
    assert L.fmha_fwd_run(ctypes.byref(a), None) == _lib.ERR_INVALID_ARG
    a = batch_args()
    a.lse = None
    assert L.fmha_fwd_run(ctypes.byref(a), None) == _lib.ERR_INVALID_ARG
    a = batch_args()
    a.q = FAKE + 8
    assert L.fmha_fwd_run(ctypes.byref(a), None) == _lib.ERR_UNSUPPORTED
    a = batch_args()
    a.scale = 0.0
    assert L.fmha_fwd_run(ctypes.byref(a), None) == _lib.ERR_UNSUPPORTED


def test_bf16_accumulator_plan():
    """bf16 accumulation: one zeroed bf16 slot per (segment, head) of the longest segment's
    rows rounded up to the query block, indexed by logical position, whatever the physical
    layout."""
    a = batch_args(deterministic=0)
    a.dq_acc_dtype = _lib.DQ_ACC_BF16
    info = _lib.plan_query(a)
    assert _lib.workspace_size(a) == info.workspace_bytes
    assert (info.nsplits, info.needs_zero, info.dq_acc_elem_bytes) == (1, 1, 2)
    assert info.tile_m == 64 and info.acc_rows == 256  # Sq = 200 rounded up to 64
    assert info.dq_acc_bytes == 2 * 4 * 256 * 128 * 2
    lens = [103, 77, 61]
    g = group_args(lens, lens, deterministic=0)
    g.dq_acc_dtype = _lib.DQ_ACC_BF16
    pq = np.array([0, 112, 192, 256], np.int32)
    g.seqstart_q_padded_host = pq.ctypes.data
    g.seqstart_q_padded_dev = FAKE
    g._keep2 = pq
    info = _lib.plan_query(g)
    assert info.rows_q == 256 and info.acc_rows == 128  # 103 -> 128
    assert info.dq_acc_bytes == 3 * 4 * 128 * 128 * 2
    assert info.dq_acc_offset + info.dq_acc_bytes <= info.workspace_bytes
    assert _lib.plan_query(batch_args(deterministic=0)).dq_acc_elem_bytes == 4


def _with_bias(a, bb, bh, dbias=True):
    Sq, Sk = a.Sq, a.Sk
    a.bias = FAKE
    a.bias_b, a.bias_h = bb, bh
    a.bias_stride[0], a.bias_stride[1], a.bias_stride[2] = bh * Sq * 336, Sq * 336, 336
    if dbias:
        a.dbias = FAKE
        a.dbias_stride[0], a.dbias_stride[1], a.dbias_stride[2] = bh * Sq * 336, Sq * 336, 336
    return a


def test_bias_plan():
    """A bias of shape (1|B, 1|Hq, Sq, Sk): dbias needs an fp32 full-shape dS region in the
    workspace; d_qk = 128 then uses 32-row query blocks."""
    for bb, bh in ((1, 1), (1, 4), (2, 1), (2, 4)):
        a = _with_bias(batch_args(), bb, bh)
        info = _lib.plan_query(a)
        assert info.tile_m == 32
        # a full-shape dbias is written directly; broadcast shapes sum an fp32 full-shape dS
        assert info.dbias_acc_bytes == (0 if (bb, bh) == (2, 4) else 2 * 4 * 200 * 333 * 4)
        assert info.dbias_acc_offset % 256 == 0
        assert info.dbias_acc_offset >= info.dq_acc_offset + info.dq_acc_bytes
        assert info.dbias_acc_offset + info.dbias_acc_bytes <= info.workspace_bytes
        assert _lib.workspace_size(a) == info.workspace_bytes
    a = _with_bias(batch_args(), 1, 1, dbias=False)
    info = _lib.plan_query(a)
    assert info.dbias_acc_bytes == 0
    assert _lib.plan_query(batch_args()).tile_m == 64


@pytest.mark.parametrize("mutate,expected", [
    (lambda a: setattr(a, "bias_b", 3), _lib.ERR_INVALID_ARG),
    (lambda a: setattr(a, "bias_h", 2), _lib.ERR_INVALID_ARG),
    (lambda a: setattr(a, "bias", FAKE + 1), _lib.ERR_UNSUPPORTED),  # not bf16-aligned
    (lambda a: a.bias_stride.__setitem__(2, 332), _lib.ERR_UNSUPPORTED),  # row stride < Sk
    (lambda a: a.dbias_stride.__setitem__(2, 332), _lib.ERR_UNSUPPORTED),
    (lambda a: setattr(a, "dbias", FAKE + 1), _lib.ERR_UNSUPPORTED),
    (lambda a: setattr(a, "bias", None), _lib.ERR_INVALID_ARG),  # dbias without a bias
])
def test_bias_argument_errors(mutate, expected):
    a = _with_bias(batch_args(), 2, 4)
    assert status_of(a) == _lib.OK
    mutate(a)
    assert status_of(a) == expected


def test_bias_row_stride_may_be_any_value_at_least_sk():
    a = _with_bias(batch_args(), 2, 4)
    a.bias_stride[2] = 333
    a.dbias_stride[2] = 335
    assert status_of(a) == _lib.OK


@pytest.mark.parametrize("p,expected", [(0.0, 0), (0.1, 0), (0.5, 0), (0.998, 0), (0.999, -2),
                                          (1.0, -1), (-0.1, -1), (float("nan"), -1)])
def test_dropout_probability_range(p, expected):
    """p_drop in [0, 1) with a keep threshold round((1-p)*256) of at least 1."""
    a = batch_args()
    a.p_drop = p
    assert status_of(a) == expected


def test_block_rows_with_bias_and_dropout_at_d128():
    """A bias at d_qk = 128 takes 32-row query blocks unless the main kernel can stage it in
    16-byte chunks; dropout alone keeps 64."""
    a = batch_args()
    a.p_drop = 0.1
    assert _lib.plan_query(a).tile_m == 64
    a = _with_bias(batch_args(), 1, 1, dbias=False)
    a.p_drop = 0.1
    assert _lib.plan_query(a).tile_m == 32
    # 64-row blocks where the kernel stages the bias in 16-byte chunks: rows 16-byte aligned
    # (pointer and every stride of a non-broadcast dimension a multiple of 8) and Sk % 8 == 0
    for bb, bh in ((1, 1), (2, 4)):
        st = _with_bias(batch_args(Sk=336), bb, bh, dbias=False)
        assert _lib.plan_query(st).tile_m == 64
        st.tune_tile_m = 32
        assert _lib.plan_query(st).tile_m == 32
    odd = _with_bias(batch_args(Sk=336), 2, 4, dbias=False)
    odd.bias_stride[0] += 4  # a batch stride that breaks 16-byte rows
    assert _lib.plan_query(odd).tile_m == 32
    odd.tune_tile_m = 64
    assert status_of(odd) == _lib.ERR_INVALID_ARG
    bcast = _with_bias(batch_args(Sk=336), 1, 1, dbias=False)
    bcast.bias_stride[0] += 4  # broadcast dimensions' strides do not matter
    assert _lib.plan_query(bcast).tile_m == 64
    moved = _with_bias(batch_args(Sk=336), 1, 1, dbias=False)
    moved.bias = FAKE + 8
    assert _lib.plan_query(moved).tile_m == 32


def test_block_rows_by_head_dim():
    """128-row query blocks at d_qk = 64 (64 with a bias or fp32 dQ atomics), 64 at 128, 32
    at 192; the deterministic accumulator pads each segment by one block."""
    def plan(dqk, dv, bias=False, det=1, bf16=False):
        a = batch_args(d_qk=dqk, d_v=dv, deterministic=det)
        if bf16:
            a.dq_acc_dtype = _lib.DQ_ACC_BF16
        return _lib.plan_query(_with_bias(a, 1, 1, dbias=False) if bias else a)
    assert plan(64, 64).tile_m == 128
    assert plan(64, 64, det=0, bf16=True).tile_m == 128
    assert plan(64, 64, det=0).tile_m == 64  # fp32 atomics
    assert plan(64, 64, bias=True).tile_m == 64
    assert plan(128, 128).tile_m == 64
    assert plan(192, 128).tile_m == 32
    info = plan(64, 64)
    assert info.acc_rows == info.rows_q + 2 * 128  # two batch entries, one block of padding each


def test_bias_needs_batch_mode():
    g = group_args([5, 7], [5, 7])
    g.bias = FAKE
    g.bias_b, g.bias_h = 1, 1
    g.bias_stride[2] = 8
    assert status_of(g) == _lib.ERR_UNSUPPORTED


def test_reduce_read_bytes_closed_forms():
    """Causal 4096 with 64-row blocks and items of 4 key tiles: block qb is touched by key tiles
    0 .. qb/2, i.e. splits 0 .. qb/8, so 288 split reads of 32 KiB per head; the atomic modes
    read the segment rows once (fp32, or bf16)."""
    a = batch_args(B=2, Hq=32, Hkv=32, Sq=4096, Sk=4096, mask=1)
    assert _lib.plan_query(a).reduce_read_bytes == 64 * 288 * 64 * 128 * 4
    a = batch_args(B=2, Hq=32, Hkv=32, Sq=4096, Sk=4096, mask=1, deterministic=0)
    assert _lib.plan_query(a).reduce_read_bytes == 2 * 32 * 4096 * 128 * 4
    a.dq_acc_dtype = _lib.DQ_ACC_BF16
    assert _lib.plan_query(a).reduce_read_bytes == 2 * 32 * 4096 * 128 * 2
    n = batch_args(B=1, Hq=2, Hkv=2, Sq=256, Sk=512, mask=0)  # no mask: every split, 4 blocks
    info = _lib.plan_query(n)
    assert info.reduce_read_bytes == 2 * 4 * info.nsplits * 64 * 128 * 4


def test_kv_parts_fill_the_gpu_for_few_heads():
    """Fewer than 256 (K/V head, key tile) items: each item's steps are split over parts of
    ceil(512 / items) work groups (at most 8), with an fp32 dK/dV partial region of parts x
    Hkv x rows_k x (d_qk + d_v).  Deterministic items keep the largest of 4 and 2 tiles for
    which 8 parts still make 512 work groups; the other modes use one tile per item."""
    shard = batch_args(B=1, Hq=4, Hkv=1, Sq=16384, Sk=16384, mask=2)  # 128 key tiles, one K/V head
    info = _lib.plan_query(shard)
    assert (info.kv_parts, info.tiles_per_item, info.nsplits) == (8, 2, 64)
    assert info.dkv_acc_bytes == 8 * 1 * 16384 * 256 * 4
    assert info.dkv_acc_offset % 256 == 0 and info.dkv_acc_offset + info.dkv_acc_bytes <= info.workspace_bytes
    shard.deterministic = 0
    info = _lib.plan_query(shard)
    assert (info.kv_parts, info.tiles_per_item) == (4, 1)
    head = _lib.plan_query(batch_args(B=2, Hq=32, Hkv=32, Sq=4096, Sk=4096, mask=1))
    assert (head.kv_parts, head.dkv_acc_bytes) == (1, 0)
    small = batch_args()  # 3 key tiles x 4 heads: one tile per item, parts capped at 8
    assert (_lib.plan_query(small).kv_parts, _lib.plan_query(small).tiles_per_item) == (8, 1)
    small.tune_tiles_per_item = 2  # the overrides apply independently
    assert (_lib.plan_query(small).kv_parts, _lib.plan_query(small).tiles_per_item) == (8, 2)
    small.tune_kv_parts = 3
    assert (_lib.plan_query(small).kv_parts, _lib.plan_query(small).tiles_per_item) == (3, 2)


def test_plan_reads_only_its_arguments(monkeypatch):
    """The plan is a pure function of the argument struct (and the host seqstart arrays): the
    environment variables that once tuned it change nothing between the sizing, prepare and
    run calls ("[ROCm] Fix THD/ragged dQ backward on the bf16 dq_shuffle path (gfx950)", Root
    cause: a sizing pass that disagreed with the run)."""
    for kernel in (_lib.KERNEL_AUTO, _lib.KERNEL_FOUR_WAVE):
        a = batch_args(B=2, Hq=16, Hkv=16, Sq=2048, Sk=2048, mask=1, kernel=kernel)
        size = _lib.workspace_size(a)
        before = _lib.plan_query(a).as_dict()
        for name, val in (("FMHA_BWD_TILE_M", "32"), ("FMHA_BWD_TILES_PER_ITEM", "4"),
                          ("FMHA_BWD_KV_PARTS", "3")):
            monkeypatch.setenv(name, val)
        assert _lib.plan_query(a).as_dict() == before
        assert _lib.workspace_size(a) == size


def test_wide_kernel_plan():
    """d_qk = d_v = 128 or 64 without bias or dropout runs the eight-wave kernel: 256-key tiles
    and 32-row query blocks; the deterministic and bf16 accumulators follow that block height."""
    for d in (128, 64):
        for det, acc in ((1, _lib.DQ_ACC_FP32), (0, _lib.DQ_ACC_FP32), (0, _lib.DQ_ACC_BF16)):
            a = batch_args(B=2, Hq=4, Hkv=2, Sq=200, Sk=333, d_qk=d, d_v=d, deterministic=det,
                           kernel=_lib.KERNEL_AUTO)
            a.dq_acc_dtype = acc
            info = _lib.plan_query(a)
            assert (info.kernel, info.tile_m, info.tile_n) == (_lib.KERNEL_WIDE, 32, 256)
            assert info.n_kv_tiles == 2 and info.n_q_blocks == 7
            assert _lib.workspace_size(a) == info.workspace_bytes
            if det:
                assert info.acc_rows == 2 * 200 + 2 * 32 and info.nsplits == 2
                assert info.dq_acc_bytes == 2 * 4 * info.acc_rows * d * 4
            elif acc == _lib.DQ_ACC_BF16:
                assert info.acc_rows == 224  # 200 rounded up to 32
    # d_qk = 192, a bias, or an explicit request keep the four-wave kernel
    assert _lib.plan_query(batch_args(d_qk=192, d_v=128, kernel=_lib.KERNEL_AUTO)).kernel == _lib.KERNEL_FOUR_WAVE
    four = batch_args(d_qk=64, d_v=64, kernel=_lib.KERNEL_FOUR_WAVE)
    assert (_lib.plan_query(four).kernel, _lib.plan_query(four).tile_m) == (_lib.KERNEL_FOUR_WAVE, 128)
    drop = batch_args(kernel=_lib.KERNEL_AUTO)  # dropout runs in the wide kernel too
    drop.p_drop = 0.1
    assert _lib.plan_query(drop).kernel == _lib.KERNEL_WIDE
    assert _lib.plan_query(batch_args()).kernel == _lib.KERNEL_FOUR_WAVE
    # a query head's rows of a whole segment must stay inside 32-bit offsets for the wide
    # kernel: (Sq + 32) * 4096 elements of sequence stride reaches 2^30 at Sq = 262112
    ok = batch_args(B=1, Hq=32, Hkv=8, Sq=262112 - 1, Sk=256, kernel=_lib.KERNEL_AUTO)
    assert _lib.plan_query(ok).kernel == _lib.KERNEL_WIDE
    long_q = batch_args(B=1, Hq=32, Hkv=8, Sq=262112, Sk=256, kernel=_lib.KERNEL_AUTO)
    assert _lib.plan_query(long_q).kernel == _lib.KERNEL_FOUR_WAVE
    long_q.tune_kernel = _lib.KERNEL_WIDE
    assert status_of(long_q) == _lib.ERR_INVALID_ARG
    # the wide kernel cannot be forced where it does not apply; its block height is fixed
    bad = batch_args(d_qk=192, d_v=128, kernel=_lib.KERNEL_WIDE)
    assert status_of(bad) == _lib.ERR_INVALID_ARG
    bad = batch_args(kernel=_lib.KERNEL_WIDE)
    bad.tune_tile_m = 64
    assert status_of(bad) == _lib.ERR_INVALID_ARG
    for field, val in (("tune_kernel", 3), ("tune_tiles_per_item", 3), ("tune_kv_parts", 9),
                       ("tune_kv_parts", -1)):
        a = batch_args()
        setattr(a, field, val)
        assert status_of(a) == _lib.ERR_INVALID_ARG, field


def test_wide_plan_splits_uneven_items():
    """Wide layout: two parts when the heaviest (segment, K/V head, key tile) item has more
    than 1.6x the steps a CU would get from a perfect split and the items average 64 steps or
    more; long causal rows take 4-tile items in parts that make about 512 work groups."""
    auto = _lib.KERNEL_AUTO
    random_8192 = [1673, 226, 413, 527, 417, 1652, 1788, 1496]
    mixed_8192 = [100, 80, 76, 200, 56, 1673, 226, 413, 527, 417, 1652, 1788, 984]
    for lens in (random_8192, mixed_8192):
        for det, acc in ((1, _lib.DQ_ACC_FP32), (0, _lib.DQ_ACC_FP32), (0, _lib.DQ_ACC_BF16)):
            a = group_args(lens, lens, Hq=32, Hkv=8, mask=1, deterministic=det, kernel=auto)
            a.dq_acc_dtype = acc
            info = _lib.plan_query(a)
            assert info.kernel == _lib.KERNEL_WIDE
            assert (info.kv_parts, info.tiles_per_item) == (2, 1), (lens[0], det, acc)
            assert info.dkv_acc_bytes == 2 * 8 * 8192 * 256 * 4
    # 2x16x2048 causal: items of 36 steps on average keep one part
    for det in (1, 0):
        info = _lib.plan_query(batch_args(B=2, Hq=16, Hkv=16, Sq=2048, Sk=2048, mask=1,
                                          deterministic=det, kernel=auto))
        assert (info.kv_parts, info.tiles_per_item) == (1, 1)
    info = _lib.plan_query(batch_args(B=2, Hq=32, Hkv=32, Sq=4096, Sk=4096, mask=1, kernel=auto))
    assert (info.kv_parts, info.tiles_per_item, info.nsplits) == (1, 2, 8)
    c4 = batch_args(B=1, Hq=32, Hkv=8, Sq=16384, Sk=16384, mask=2, kernel=auto)
    info = _lib.plan_query(c4)
    assert (info.kv_parts, info.tiles_per_item, info.nsplits) == (4, 4, 16)
    c4.deterministic = 0
    assert _lib.plan_query(c4).kv_parts == 1
    w = batch_args(B=1, Hq=32, Hkv=8, Sq=16384, Sk=16384, mask=3, window=(4096, 0), kernel=auto)
    assert (_lib.plan_query(w).kv_parts, _lib.plan_query(w).tiles_per_item) == (1, 2)


def test_ragged_wide_plans_order_their_work_groups():
    """Ragged batches in the wide layout take a longest-first list of the main kernel's work
    groups (written by prepare at the end of the workspace); batch mode, the four-wave layout
    and grids of more than 2048 work groups keep the grid order."""
    auto = _lib.KERNEL_AUTO
    lens = [1673, 226, 413, 527, 417, 1652, 1788, 1496]
    for det in (1, 0):
        a = group_args(lens, lens, Hq=32, Hkv=8, mask=1, deterministic=det, kernel=auto)
        info = _lib.plan_query(a)
        wgs = -(-info.n_kv_tiles // info.tiles_per_item) * info.kv_parts * 8 * len(lens)
        assert info.ordered_groups == wgs == 7 * 2 * 8 * 8
        assert info.workspace_bytes >= info.dkv_acc_offset + info.dkv_acc_bytes + 4 * wgs
        assert _lib.workspace_size(a) == info.workspace_bytes
    assert _lib.plan_query(group_args(lens, lens, Hq=32, Hkv=8, mask=1)).ordered_groups == 0  # four-wave
    assert _lib.plan_query(batch_args(B=2, Hq=32, Hkv=32, Sq=4096, Sk=4096, mask=1, kernel=auto)).ordered_groups == 0
    many = group_args([2048] * 200, [2048] * 200, Hq=32, Hkv=8, mask=1, kernel=auto)
    info = _lib.plan_query(many)  # 2 items of 4 tiles x 8 K/V heads x 200 segments > 2048
    assert info.tiles_per_item == 4 and info.ordered_groups == 0


def test_bf16_accumulator_tile_limit():
    """bf16 accumulation adds one rounded contribution per key tile; the plan refuses more than
    64 tiles per segment, where the error estimate u*sqrt(n/6) (u = 2^-8) leaves the cosine
    bar, instead of returning a dQ outside it."""
    for kernel, tile_n in ((_lib.KERNEL_AUTO, 256), (_lib.KERNEL_FOUR_WAVE, 128)):
        ok = batch_args(B=1, Hq=4, Hkv=4, Sq=256, Sk=64 * tile_n, deterministic=0, kernel=kernel)
        ok.dq_acc_dtype = _lib.DQ_ACC_BF16
        assert _lib.plan_query(ok).n_kv_tiles == 64
        over = batch_args(B=1, Hq=4, Hkv=4, Sq=256, Sk=64 * tile_n + 1, deterministic=0, kernel=kernel)
        over.dq_acc_dtype = _lib.DQ_ACC_BF16
        assert status_of(over) == _lib.ERR_UNSUPPORTED
        over.dq_acc_dtype = _lib.DQ_ACC_FP32
        assert status_of(over) == _lib.OK


def test_tiles_per_item_keeps_two_items_per_cu():
    """Deterministic work items take 4 key tiles when that leaves >= 512 items, else 2, else 1;
    the split count follows.  Causal segments of 8192 keys or more whose 4-tile items number
    256 to 511 take 4 tiles split into parts (at most 4) that make about 1024 work groups."""
    for B, H, S, want, parts in ((2, 32, 4096, 4, 1), (1, 8, 16384, 4, 4), (1, 12, 16384, 4, 3),
                                 (1, 8, 8192, 1, 1), (2, 16, 2048, 1, 1)):
        a = batch_args(B=B, Hq=H, Hkv=H, Sq=S, Sk=S, mask=1)
        info = _lib.plan_query(a)
        tiles = -(-S // 128)
        assert (info.tiles_per_item, info.kv_parts) == (want, parts), (B, H, S)
        assert info.nsplits == -(-tiles // want)
    a = batch_args(B=2, Hq=32, Hkv=32, Sq=4096, Sk=4096, mask=1, deterministic=0)
    assert _lib.plan_query(a).tiles_per_item == 1
    # a two-sided window (even work per tile) needs one item per compute unit only
    w = batch_args(B=1, Hq=32, Hkv=8, Sq=16384, Sk=16384, mask=3, window=(4096, 0))
    assert _lib.plan_query(w).tiles_per_item == 4
    assert _lib.plan_query(w).kv_parts == 1
    c = batch_args(B=1, Hq=32, Hkv=8, Sq=16384, Sk=16384, mask=2)
    assert (_lib.plan_query(c).tiles_per_item, _lib.plan_query(c).kv_parts) == (4, 4)
    c.deterministic = 0
    assert (_lib.plan_query(c).tiles_per_item, _lib.plan_query(c).kv_parts) == (1, 1)


def test_scale_must_be_positive():
    for sc in (0.0, -0.125):
        a = batch_args()
        a.scale = sc
        assert status_of(a) == _lib.ERR_UNSUPPORTED
    a = batch_args()
    a.scale = float("nan")
    assert status_of(a) == _lib.ERR_INVALID_ARG


def test_padded_thd_plan():
    """Padded slots: the physical row count comes from the padded q offsets; a segment that
    does not fit its slot, a host array without its device twin, or padding in batch mode
    are argument errors."""
    lens = [103, 77, 61]
    a = group_args(lens, lens)
    pq = np.array([0, 112, 192, 256], np.int32)
    a.seqstart_q_padded_host = pq.ctypes.data
    a.seqstart_q_padded_dev = FAKE
    a.seqstart_k_padded_host = pq.ctypes.data
    a.seqstart_k_padded_dev = FAKE
    a._keep2 = pq
    info = _lib.plan_query(a)
    assert info.rows_q == 256
    assert info.pairs == sum(n * (n + 1) // 2 for n in lens) * 4  # logical lengths, causal, 4 heads
    bad = np.array([0, 100, 192, 256], np.int32)  # 103 rows do not fit a 100-row slot
    a.seqstart_q_padded_host = bad.ctypes.data
    a._keep3 = bad
    assert status_of(a) == _lib.ERR_INVALID_ARG
    a.seqstart_q_padded_host = pq.ctypes.data
    a.seqstart_q_padded_dev = None
    assert status_of(a) == _lib.ERR_INVALID_ARG
    b = batch_args()
    b.seqstart_q_padded_host = pq.ctypes.data
    b.seqstart_q_padded_dev = FAKE
    b._keep = pq
    assert status_of(b) == _lib.ERR_INVALID_ARG


def test_flop_count_matches_pair_count():
    a = batch_args(B=2, Hq=16, Hkv=16, Sq=2048, Sk=2048, mask=1)
    info = _lib.plan_query(a)
    pairs = 2 * 16 * 2048 * 2049 // 2
    assert info.pairs == pairs
    assert info.flops == 2.0 * (3 * 128 + 2 * 128) * pairs
    w = batch_args(B=1, Hq=1, Hkv=1, Sq=16384, Sk=16384, mask=3, window=(4096, 0))
    assert _lib.plan_query(w).pairs == 58734592  # 4097 keys per row, fewer near the start


@pytest.mark.parametrize("mutate,expected", [
    (lambda a: setattr(a, "struct_size", 8), _lib.ERR_INVALID_ARG),
    (lambda a: setattr(a, "abi_version", 99), _lib.ERR_INVALID_ARG),
    (lambda a: setattr(a, "Hkv", 3), _lib.ERR_INVALID_ARG),
    (lambda a: setattr(a, "d_qk", 96), _lib.ERR_UNSUPPORTED),
    (lambda a: (setattr(a, "d_qk", 128), setattr(a, "d_v", 64)), _lib.ERR_UNSUPPORTED),
    (lambda a: setattr(a, "mask_type", 7), _lib.ERR_INVALID_ARG),
    (lambda a: setattr(a, "window_left", 5), _lib.ERR_INVALID_ARG),  # NONE with a window
    (lambda a: setattr(a, "scale", float("nan")), _lib.ERR_INVALID_ARG),
    (lambda a: setattr(a, "q", 0), _lib.ERR_INVALID_ARG),
    (lambda a: setattr(a, "q", FAKE + 8), _lib.ERR_UNSUPPORTED),
    (lambda a: a.q_stride.__setitem__(1, 4 * 128 + 4), _lib.ERR_UNSUPPORTED),
    (lambda a: setattr(a, "deterministic", 2), _lib.ERR_INVALID_ARG),
    (lambda a: setattr(a, "dq_acc_dtype", 1), _lib.ERR_INVALID_ARG),  # bf16 needs atomic mode
    (lambda a: setattr(a, "dq_acc_dtype", 2), _lib.ERR_INVALID_ARG),
    (lambda a: setattr(a, "reserved", 1), _lib.ERR_INVALID_ARG),
    (lambda a: setattr(a, "B", -1), _lib.ERR_INVALID_ARG),
    (lambda a: setattr(a, "seqstart_k_host", FAKE), _lib.ERR_INVALID_ARG),  # half group mode
])
def test_invalid_arguments_are_rejected(mutate, expected):
    a = batch_args()
    assert status_of(a) == _lib.OK
    mutate(a)
    assert status_of(a) == expected


def test_group_mode_errors():
    a = group_args([5, 7], [5, 7])
    assert status_of(a) == _lib.OK
    a.seqstart_q_dev = 0  # device offsets missing
    assert status_of(a) == _lib.ERR_INVALID_ARG
    bad = group_args([5, 7], [5, 7])
    bad._keep[0][2] = 3  # non-monotone
    assert status_of(bad) == _lib.ERR_INVALID_ARG
    long = group_args([5, 7], [5, 7])
    long.Sq = 6  # a segment longer than the declared maximum
    assert status_of(long) == _lib.ERR_INVALID_ARG


def test_window_masks_need_window_type():
    assert status_of(batch_args(mask=3, window=(10, 0))) == _lib.OK
    assert status_of(batch_args(mask=1, window=(10, 0))) == _lib.ERR_INVALID_ARG
    assert status_of(batch_args(mask=3, window=(-2, 0))) == _lib.ERR_INVALID_ARG


def test_workspace_too_small_is_reported_before_any_device_work():
    a = batch_args()
    n = _lib.workspace_size(a)
    L = _lib.lib()
    st = L.fmha_bwd_run(ctypes.byref(a), ctypes.c_void_p(FAKE), n - 1, None)
    assert st == _lib.ERR_WORKSPACE_TOO_SMALL
    st = L.fmha_bwd_prepare_workspace(ctypes.byref(a), ctypes.c_void_p(FAKE), n - 1, None)
    assert st == _lib.ERR_WORKSPACE_TOO_SMALL
    st = L.fmha_bwd_run_stages(ctypes.byref(a), ctypes.c_void_p(FAKE), n, 8, None)
    assert st == _lib.ERR_INVALID_ARG
    assert _lib.status_string(_lib.ERR_WORKSPACE_TOO_SMALL) == "FMHA_ERR_WORKSPACE_TOO_SMALL"


def test_noalloc_rejects_arguments_beyond_its_scratch_before_any_device_work():
    a = batch_args(B=2, Hq=32, Hkv=32, Sq=4096, Sk=4096, mask=1, deterministic=1,
                   kernel=_lib.KERNEL_AUTO)
    assert _lib.workspace_size(a) > _lib.NOALLOC_MAX_BYTES
    assert _lib.lib().fmha_bwd_run_noalloc(ctypes.byref(a), None) == _lib.ERR_WORKSPACE_TOO_SMALL
    a.Hq = 3  # invalid arguments are reported as such
    assert _lib.lib().fmha_bwd_run_noalloc(ctypes.byref(a), None) == _lib.ERR_INVALID_ARG
    m = re.search(r"#define FMHA_BWD_NOALLOC_MAX_BYTES \((\d+)u << (\d+)\)", open(HEADER).read())
    assert m and int(m.group(1)) << int(m.group(2)) == _lib.NOALLOC_MAX_BYTES


def test_sizing_is_a_pure_function_of_the_arguments():
    """The same arguments always give the same plan, and only the fields that define the
    problem change it (pointer values do not)."""
    rng = np.random.default_rng(5)
    for _ in range(200):
        nseg = int(rng.integers(1, 6))
        lq = rng.integers(0, 700, nseg)
        lk = rng.integers(0, 700, nseg)
        if lq.sum() == 0 or lk.sum() == 0:
            continue
        d = int(rng.choice([64, 128, 192]))
        det = int(rng.integers(0, 2))
        a = group_args(list(lq), list(lk), Hq=4, Hkv=int(rng.choice([1, 2, 4])), d=d, mask=int(rng.integers(0, 3)),
                       deterministic=det)
        if d == 192:
            a.d_v = 128
        i1 = _lib.plan_query(a).as_dict()
        a.q = FAKE * 3
        a.dq = FAKE * 5
        i2 = _lib.plan_query(a).as_dict()
        assert i1 == i2
        assert i1["workspace_bytes"] == _lib.workspace_size(a)
        nt = -(-int(lk.max()) // i1["tile_n"])
        assert i1["n_kv_tiles"] == nt
        tpi = i1["tiles_per_item"]
        assert tpi in ((1, 2, 4) if det else (1,))
        assert i1["nsplits"] == (max(-(-nt // tpi), 1) if det else 1)
        assert i1["rows_q"] == int(lq.sum())
