"""Writes segments.json: the ragged segment packings used by the THD tests and benchmark.

Fixed packings are cited from "[ROCm] Fix THD/ragged dQ backward on the bf16 dq_shuffle path
(gfx950)": [256], [100,80,76], [128,128], [64,64,64,64], [200,56] (Verification) and
[103,77,61] plus a 2044-long segment (review replies).  The seeded ones come from
``attention_backward_fmha_amd.inputs.ragged_lengths`` (seed 3, lengths in [56, 2048],
8192 tokens in all).  Stored so that a numpy version change can never alter them.
Run: python tests/golden/make_segments.py
"""
import json
import os
import sys

sys.path.insert(0, os.path.join(os.path.dirname(os.path.abspath(__file__)), "..", ".."))
from attention_backward_fmha_amd.inputs import ragged_lengths  # noqa: E402

out = {
    "fixed_from_pages": {
        "single_256": [256],
        "split_100_80_76": [100, 80, 76],
        "split_128_128": [128, 128],
        "split_64x4": [64, 64, 64, 64],
        "split_200_56": [200, 56],
        "split_103_77_61": [103, 77, 61],
        "single_2044": [2044],
    },
    "random_8192": ragged_lengths(3, 8192, 56, 2048),
    "mixed_8192": ragged_lengths(3, 8192, 56, 2048, prefix=(100, 80, 76, 200, 56)),
}
path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "segments.json")
with open(path, "w") as f:
    json.dump(out, f, indent=1)
print(path)
