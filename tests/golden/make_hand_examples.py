"""Writes hand_examples.json: small attention problems solved by hand in closed form.

The pages print no worked numeric example, so these fixtures are derived by
hand from the definition they state and are evaluated here to 40 significant
digits with Python's ``decimal`` module (no floating point, no oracle, no GPU):

  "Understand FlashAttention" (nothiny.github.io), section "前向传播":
  S = Q K^T, P = softmax(S), O = P V; section "附：数值稳定的logsumexp(L)推导":
  L_i = log sum_j e^{S_ij}.  "PyTorch profiling part 3: attention", section
  "朴素注意力": the scores are multiplied by the scale after Q K^T and masked
  entries (causal: key j > query i, "构建因果掩码" builds the lower triangle)
  are set to -inf before the softmax.

Every input is a small integer (or ln 3 in one case), so each score is a
closed-form number and each output is a ratio of sums of exponentials.

Run:  python tests/golden/make_hand_examples.py
"""
from __future__ import annotations

import json
import os
from decimal import Decimal, getcontext

getcontext().prec = 50
E = Decimal(1).exp()


def D(x) -> Decimal:
    return Decimal(x)


def s40(x: Decimal) -> str:
    return format(+x.normalize(), ".40g") if x != 0 else "0"


def example_causal_two_keys():
    # q = [[1],[1]], k = [[0],[ln 3]], v = [[4],[8]], scale 1, causal.
    # row 0 sees key 0 only: o_0 = v_0 = 4, lse_0 = s_00 = 0.
    # row 1: s = [0, ln 3] -> weights [1, 3] / 4 -> o_1 = (4 + 24)/4 = 7, lse_1 = ln 4.
    ln3 = D(3).ln()
    return {
        "name": "causal_two_keys",
        "cite": "Understand FlashAttention, section 前向传播 (O = softmax(Q K^T) V) and the "
                "logsumexp appendix; PyTorch profiling part 3, section 构建因果掩码 (lower triangle).",
        "derivation": "row0: only key 0 allowed -> o=v0=4, lse=s00=0; row1: s=[0, ln3], "
                      "P=[1/4, 3/4], o=1+6=7, lse=ln(1+3)=ln4",
        "scale": 1.0, "causal": True,
        "q": [[1.0], [1.0]], "k": [[0.0], [float(ln3)]], "v": [[4.0], [8.0]],
        "o": [["4"], ["7"]],
        "lse": ["0", s40(D(4).ln())],
    }


def example_noncausal_three_keys():
    # q = [[2,0],[0,2],[2,2]], k = [[0,0],[2,0],[0,2]], scale 1/2
    # s = q k^T / 2: row0 [0,2,0], row1 [0,0,2], row2 [0,2,2].
    e2 = E ** 2
    z01 = 2 + e2
    z2 = 1 + 2 * e2
    o0 = [D(2) / z01, (1 + e2) / z01]            # (v0 + e^2 v1 + v2) / (2 + e^2)
    o1 = [(1 + e2) / z01, (1 + e2) / z01]        # (v0 + v1 + e^2 v2) / (2 + e^2)
    o2 = [(1 + e2) / z2, (2 * e2) / z2]          # (v0 + e^2 v1 + e^2 v2) / (1 + 2 e^2)
    return {
        "name": "noncausal_three_keys",
        "cite": "Understand FlashAttention, section 前向传播 and the logsumexp appendix; "
                "PyTorch profiling part 3, section 朴素注意力 (scale after Q K^T).",
        "derivation": "s=[[0,2,0],[0,0,2],[0,2,2]]; v=[[1,0],[0,1],[1,1]]; "
                      "o0=[2,1+e^2]/(2+e^2); o1=[1+e^2,1+e^2]/(2+e^2); "
                      "o2=[1+e^2,2e^2]/(1+2e^2); lse=[ln(2+e^2), ln(2+e^2), ln(1+2e^2)]",
        "scale": 0.5, "causal": False,
        "q": [[2.0, 0.0], [0.0, 2.0], [2.0, 2.0]],
        "k": [[0.0, 0.0], [2.0, 0.0], [0.0, 2.0]],
        "v": [[1.0, 0.0], [0.0, 1.0], [1.0, 1.0]],
        "o": [[s40(x) for x in o0], [s40(x) for x in o1], [s40(x) for x in o2]],
        "lse": [s40(z01.ln()), s40(z01.ln()), s40(z2.ln())],
    }


def example_causal_three_keys():
    # Same q, k, v as above, causal: row0 sees key 0; row1 keys 0,1; row2 keys 0..2.
    # row0: o=v0=[1,0], lse=0.  row1: s=[0,0] -> o=(v0+v1)/2=[1/2,1/2], lse=ln2.
    # row2: s=[0,2,2] -> as the non-causal row 2.
    e2 = E ** 2
    z2 = 1 + 2 * e2
    return {
        "name": "causal_three_keys",
        "cite": "PyTorch profiling part 3, sections 朴素注意力 and 构建因果掩码 (key j allowed "
                "iff j <= i); Understand FlashAttention, logsumexp appendix.",
        "derivation": "row0: o=v0, lse=s00=0; row1: s=[0,0], o=(v0+v1)/2, lse=ln2; "
                      "row2: s=[0,2,2], o=[1+e^2,2e^2]/(1+2e^2), lse=ln(1+2e^2)",
        "scale": 0.5, "causal": True,
        "q": [[2.0, 0.0], [0.0, 2.0], [2.0, 2.0]],
        "k": [[0.0, 0.0], [2.0, 0.0], [0.0, 2.0]],
        "v": [[1.0, 0.0], [0.0, 1.0], [1.0, 1.0]],
        "o": [["1", "0"], ["0.5", "0.5"], [s40((1 + e2) / z2), s40(2 * e2 / z2)]],
        "lse": ["0", s40(D(2).ln()), s40(z2.ln())],
    }


def main():
    out = {
        "about": "Hand-derived attention examples; expected values are closed forms "
                 "evaluated to 40 digits by tests/golden/make_hand_examples.py.",
        "examples": [example_causal_two_keys(), example_noncausal_three_keys(),
                     example_causal_three_keys()],
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "hand_examples.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(path)


if __name__ == "__main__":
    main()
