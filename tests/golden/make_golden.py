"""Writes the stored expected values under tests/golden/ by calling only the oracle.

The pages print no numeric worked example for attention, so every stored value
here is the oracle's, on seeded inputs from the synth module. Rerun with
``python tests/golden/make_golden.py`` after a justified change to the oracle.
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from oracle.attention import attention_ref, widen_bf16  # noqa: E402
from synth import make_qkv  # noqa: E402

CASES = [
    # name, B, Hq, Hkv, Sq, Skv, d, causal, seed
    ("small_causal_gqa_d64", 1, 4, 2, 19, 19, 64, True, 77),
    ("small_noncausal_d128", 1, 2, 1, 5, 70, 128, False, 78),
]


def main():
    for name, B, Hq, Hkv, Sq, Skv, d, causal, seed in CASES:
        q, k, v = make_qkv(B, Hq, Hkv, Sq, Skv, d, seed)
        scale = float(d) ** -0.5
        O, L = attention_ref(widen_bf16(q), widen_bf16(k), widen_bf16(v), causal=causal, scale=scale)
        rec = {"source": "oracle.attention.attention_ref on synth.make_qkv inputs",
               "B": B, "Hq": Hq, "Hkv": Hkv, "Sq": Sq, "Skv": Skv, "d": d, "causal": causal,
               "seed": seed, "scale": scale,
               "O": [float.hex(float(x)) for x in O.ravel()],
               "LSE": [float.hex(float(x)) for x in L.ravel()]}
        with open(os.path.join(ROOT, "tests", "golden", name + ".json"), "w") as f:
            json.dump(rec, f)
        print("wrote", name)


if __name__ == "__main__":
    main()
