"""Writes hand_example_n2_d1.json: a 2-query, 1-dim attention example whose outputs are exact
closed forms derived on paper from eq. (1)/(4)-(6), eq. (12) and eqs. (7)-(11) of the CS336
Assignment 2 (systems) handout, section 4.1, with the causal mask of Problem (flash_forward)(c).
No page prints a worked numeric example; these numbers come from the derivation below, not
from any implementation. Run: python tests/golden/make_hand_example.py
"""
import json
import math
import os

ln2, ln3 = math.log(2), math.log(3)

DERIVATION = [
    "S = q k^T = [[0, 0], [0, ln2]].",
    "non-causal: row0 P=[1/2,1/2], O=2, L=ln2; row1 exp(S)=[1,2] so P=[1/3,2/3], O=7/3, L=ln3.",
    "dV = P^T dO = [5/6, 7/6]; dP = dO v^T = [[1,3],[1,3]]; D = P.dP = [2, 7/3].",
    "dS = P o (dP - D) = [[-1/2, 1/2], [-4/9, 4/9]]; dQ = dS k = [ln2/2, 4 ln2/9]; dK = dS^T q = [-4/9, 4/9].",
    "causal: row0 keeps only key 0: P=[1,0], O=1, L=0, D_0=1, dS_0=0; row1 as above. "
    "dV=[4/3, 2/3], dQ=[0, 4 ln2/9], dK=[-4/9, 4/9].",
    "key padding kv=1 (non-causal): both rows see key 0 only: O=[1,1], L=[0,0] (S_10 = 1*0 = 0); "
    "dV=[2,0]; dQ=dK=0.",
]

CASES = {
    "noncausal": {"causal": False, "kv": None,
                  "O": [[2.0], [7 / 3]], "L": [ln2, ln3], "D": [2.0, 7 / 3],
                  "dQ": [[ln2 / 2], [4 * ln2 / 9]], "dK": [[-4 / 9], [4 / 9]], "dV": [[5 / 6], [7 / 6]]},
    "causal": {"causal": True, "kv": None,
               "O": [[1.0], [7 / 3]], "L": [0.0, ln3], "D": [1.0, 7 / 3],
               "dQ": [[0.0], [4 * ln2 / 9]], "dK": [[-4 / 9], [4 / 9]], "dV": [[4 / 3], [2 / 3]]},
    "pad_kv1": {"causal": False, "kv": 1,
                "O": [[1.0], [1.0]], "L": [0.0, 0.0], "D": [1.0, 1.0],
                "dQ": [[0.0], [0.0]], "dK": [[0.0], [0.0]], "dV": [[2.0], [0.0]]},
}

if __name__ == "__main__":
    doc = {
        "source": __doc__.strip().splitlines()[0:4],
        "inputs": {"q": [[0.0], [1.0]], "k": [[0.0], [ln2]], "v": [[1.0], [3.0]],
                   "do": [[1.0], [1.0]], "scale": 1.0},
        "derivation": DERIVATION,
        "cases": CASES,
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "hand_example_n2_d1.json")
    with open(path, "w") as f:
        json.dump(doc, f, indent=1)
