"""Writes tiny_layer_L3.json: a worked case of one prefill layer small enough to derive by hand.

The expected values are the closed forms of the derivation evaluated with the math module, with no
call into the oracle or the HIP library.  The oracle must reproduce them (tests/test_oracle_pins.py).

Definitions followed:
- papernotes.org reading notes, "Key design 2": recent-query scoring, column sums, normalised layer
  score, ascending cumulative budget, per-head top-k;
- papernotes.org reading notes, "Key design 1": gather, dense causal attention in the compressed
  space, scatter into zeros, residual;
- bxzpzcl.cn article, section 1.1: softmax(Q K^T / sqrt(d)) V.

Run from the repository root: python tests/golden/make_tiny_layer_L3.py
"""

import json
import math
import os

E = math.e

inputs = {"L": 3, "Hq": 1, "Hkv": 1, "d": 1, "q": 2, "tau": 0.1,
          "Q": [0.5, 1.0, 1.0], "K": [0.0, 1.0, 0.0], "V": [2.0, 4.0, 8.0], "X": [1.0, 1.0, 1.0]}

# recent query p = 1 sees keys 0..1 with logits (0, 1); p = 2 sees keys 0..2 with logits (0, 1, 0)
s_h = [1 / (1 + E) + 1 / (2 + E), E / (1 + E) + E / (2 + E), 1 / (2 + E)]
s_l = [v / 2 for v in s_h]                      # the column sums total q = 2
# ascending s_l: token 2 alone already reaches tau = 0.1, so k = 1 and L' = 2
k, Lp = 1, 2
idx = [0, 1]                                    # the two largest s_h, in ascending order
O_hat = [2.0, (2 + 4 * E) / (1 + E)]            # row 0 sees key 0 only; row 1 weighs (1, e)/(1 + e)
Y = [1 + O_hat[0], 1 + O_hat[1], 1 + 0.0]       # token 2 was dropped: +0.0 before the residual

doc = {
    "about": ("Hand-derived worked case of one TSA prefill layer (L=3, one head, d=1, q=2, tau=0.1). "
              "Derivation from the definitions: notes 'Key design 2' (recent-query scoring, column sum, "
              "normalised layer score, ascending cumulative budget, per-head top-k) and 'Key design 1' "
              "(gather, dense causal attention in the compressed space, scatter into zeros, residual); "
              "blog section 1.1 for softmax(QK^T/sqrt(d))V. Values are the closed forms below evaluated "
              "in double precision; e = exp(1)."),
    "inputs": inputs,
    "derivation": {
        "recent query p=1": "logits (0, 1) over keys 0..1 -> weights (1/(1+e), e/(1+e))",
        "recent query p=2": "logits (0, 1, 0) over keys 0..2 -> weights (1/(2+e), e/(2+e), 1/(2+e))",
        "s_h": ["1/(1+e) + 1/(2+e)", "e/(1+e) + e/(2+e)", "1/(2+e)"],
        "s_l": "s_h / 2 (the column sums total q = 2)",
        "budget": "ascending s_l: token 2 (0.1065...) >= tau=0.1 already -> k = 1, L' = 2",
        "select": "top-2 of s_h = tokens {1, 0} -> S = [0, 1]",
        "O_hat row 0 (pos 0)": "only key 0 visible -> V[0] = 2",
        "O_hat row 1 (pos 1)": "weights (1/(1+e), e/(1+e)) -> (2 + 4e)/(1+e)",
        "Y": "X + scatter: [1 + 2, 1 + (2+4e)/(1+e), 1 + 0]",
    },
    "expected": {"s_h": s_h, "s_l": s_l, "k": k, "Lp": Lp, "idx": idx, "O_hat": O_hat, "Y": Y},
}

if __name__ == "__main__":
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_layer_L3.json")
    with open(path, "w") as f:
        json.dump(doc, f, indent=1)
        f.write("\n")
    print("wrote", path)
