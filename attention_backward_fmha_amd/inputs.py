"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module holds no attention arithmetic: it draws random numbers, rounds them to bfloat16
and lays out ragged segment offsets.  Both the HIP path and the oracle receive what it makes.

Recipe (one per workload, see ``WORKLOADS``):
  * values: ``numpy.random.default_rng(seed)``, ``standard_normal(shape, float32) * sigma`` in
    the fixed order Q, K, V, dO, each drawn in its storage shape, then rounded to bfloat16
    (round to nearest, ties to even); the rounded values are what both sides consume;
  * ragged segment lengths: uniform integers in [lo, hi] from their own seed until what is
    left fits in one segment, which becomes the last one.
"""

import numpy as np

# Mask numbering used across the library (mirrors the mask-type table of the
# TransformerEngine PR 446 review thread on ``ck_to_aiter_mask_type``).
MASK_NONE = 0
MASK_CAUSAL_TOP_LEFT = 1
MASK_CAUSAL_BOTTOM_RIGHT = 2
MASK_WINDOW = 3


def bf16_bits(x):
    """float32 -> bfloat16 bit patterns (uint16), round to nearest, ties to even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_to_f32(bits):
    """bfloat16 bit patterns -> float32 values (exact)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)


def round_bf16(x):
    """Round float32 values to the nearest bfloat16 and return them as float32."""
    return bf16_to_f32(bf16_bits(x))


def draw(seed, shapes, sigmas=(1.0, 1.0, 1.0, 1.0)):
    """Draw Q, K, V, dO (in that order) and round them to bfloat16.

    Returns a dict name -> float32 array holding bf16-representable values."""
    rng = np.random.default_rng(seed)
    out = {}
    for name, shape, sigma in zip(("q", "k", "v", "do"), shapes, sigmas):
        x = rng.standard_normal(shape, dtype=np.float32) * np.float32(sigma)
        out[name] = round_bf16(x)
    return out


def ragged_lengths(seed, total, lo, hi, prefix=()):
    """Segment lengths summing to ``total``: the fixed ``prefix`` first, then uniform draws
    in [lo, hi]; once what is left fits in one segment (<= hi) it becomes the last one.  A
    draw that would leave less than ``lo`` is shortened so the last segment keeps >= lo."""
    rng = np.random.default_rng(seed)
    lens = [int(x) for x in prefix]
    remaining = total - sum(lens)
    while remaining > 0:
        if remaining <= hi:
            lens.append(remaining)
            break
        n = int(rng.integers(lo, hi + 1))
        if remaining - n < lo:
            n = remaining - lo
        lens.append(n)
        remaining -= n
    return lens


def seqstart(lengths):
    """Exclusive prefix sum [0, l0, l0+l1, ...] as int32."""
    return np.concatenate([[0], np.cumsum(np.asarray(lengths, np.int64))]).astype(np.int32)


# Workloads: shapes, value distributions and masks of the pages' workloads.  The segment
# packings [256], [100,80,76], [128,128], [64]*4, [200,56] come from the Verification
# section of "[ROCm] Fix THD/ragged dQ backward on the bf16 dq_shuffle path (gfx950)";
# [103,77,61] and a 2044-long segment from its review replies.  Llama-3-8B's attention head
# shape (32 query heads, 8 K/V heads, d=128) is the model named in that Verification section.
WORKLOADS = {
    "tiny": dict(B=1, Hq=1, Hkv=1, Sq=64, Sk=64, d_qk=64, d_v=64, mask=MASK_NONE, seed=1001,
                 sigmas=(1, 1, 1, 1), fp32_source=True),
    "bshd_causal_2x16x2048": dict(B=2, Hq=16, Hkv=16, Sq=2048, Sk=2048, d_qk=128, d_v=128,
                                  mask=MASK_CAUSAL_TOP_LEFT, seed=1002, sigmas=(1, 1, 1, 1)),
    "thd_gqa_llama3_8192": dict(Hq=32, Hkv=8, d_qk=128, d_v=128, total=8192, mask=MASK_CAUSAL_TOP_LEFT,
                                seed=1003, sigmas=(1, 1, 1, 1)),
    # the same tokens with the pages' fixed splits [100, 80, 76] and [200, 56] packed first
    "thd_gqa_llama3_8192_mixed": dict(Hq=32, Hkv=8, d_qk=128, d_v=128, total=8192,
                                      prefix=(100, 80, 76, 200, 56), mask=MASK_CAUSAL_TOP_LEFT,
                                      seed=1003, sigmas=(1, 1, 1, 1)),
    "long_16384_causal_br": dict(B=1, Hq=32, Hkv=8, Sq=16384, Sk=16384, d_qk=128, d_v=128,
                                 mask=MASK_CAUSAL_BOTTOM_RIGHT, seed=1004, sigmas=(1, 1, 1, 1)),
    "long_16384_window_4096": dict(B=1, Hq=32, Hkv=8, Sq=16384, Sk=16384, d_qk=128, d_v=128,
                                   mask=MASK_WINDOW, window=(4096, 0), seed=1004,
                                   sigmas=(1, 1, 1, 1)),
    # one GPU's share of the 16384-token workload under 8-way K/V-head sharding
    "long_16384_causal_shard_h4": dict(B=1, Hq=4, Hkv=1, Sq=16384, Sk=16384, d_qk=128, d_v=128,
                                       mask=MASK_CAUSAL_BOTTOM_RIGHT, seed=1004, sigmas=(1, 1, 1, 1)),
    "cross_192_128": dict(B=4, Hq=16, Hkv=16, Sq=1024, Sk=4096, d_qk=192, d_v=128, mask=MASK_NONE,
                          seed=1005, sigmas=(1, 1, 0.5, 0.5)),
    "cross_64": dict(B=4, Hq=16, Hkv=16, Sq=1024, Sk=4096, d_qk=64, d_v=64, mask=MASK_NONE,
                     seed=1006, sigmas=(1, 1, 0.5, 0.5)),
    # the throughput headline: B*H*S*d = 2*32*4096*128, causal
    "headline_2x32x4096_causal": dict(B=2, Hq=32, Hkv=32, Sq=4096, Sk=4096, d_qk=128, d_v=128,
                                      mask=MASK_CAUSAL_TOP_LEFT, seed=1007, sigmas=(1, 1, 1, 1)),
}
