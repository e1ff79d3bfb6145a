"""Writes two_key_worked_example.json: a hand-derived two-key case.

The expected values are closed forms worked out by hand from the definition
on page "Noncausal Global Extreme-GQA Ragged Attention Full VJP", section
"What You Have" (scale, soft cap, ALiBi with bottom-right alignment,
softmax) and section "Hard Constraints" (the cap acts before ALiBi).  This
script uses only the `math` module: it imports neither the oracle nor the
library.

Case: D = 4, one sequence, Lq = 1, Lk = 2, one head, scale_multiplier 0.75
(sigma = 0.75 / sqrt(4)), cap c = 3, slope mu.
  q0 = e1, k0 = x e1, k1 = 0, v0 = e1, v1 = e2, dout0 = (g0, g1, 0, 0).
Query 0 is aligned with key i + Lk - Lq = 1, so the ALiBi distances are
|1 - 0| = 1 for key 0 and 0 for key 1:
  a0 = c tanh(sigma x / c) - mu,  a1 = 0,  p = sigmoid(a0)
  out = (p, 1 - p, 0, 0),  lse = log(1 + exp(a0))
With G = (g0 - g1) p (1 - p) and T' = 1 - tanh^2(sigma x / c):
  dq  = (sigma G T' x, 0, 0, 0)
  dk0 = (sigma G T', 0, 0, 0),  dk1 = (-sigma G, 0, 0, 0)
  dv0 = p (g0, g1, 0, 0),       dv1 = (1 - p) (g0, g1, 0, 0)
The wrong order (ALiBi inside the cap) would give
p_wrong = sigmoid(c tanh((sigma x - mu) / c)); it is stored to show the case
separates the two readings.
"""
import json
import math
import os

x, mu, c, g0, g1 = 8.0, 0.5, 3.0, 0.7, -1.3
sigma = 0.75 / math.sqrt(4.0)
th = math.tanh(sigma * x / c)
a0 = c * th - mu
p = 1.0 / (1.0 + math.exp(-a0))
G = (g0 - g1) * p * (1.0 - p)
Tp = 1.0 - th * th
case = {
    "source": "hand-derived from page 'Noncausal Global Extreme-GQA Ragged Attention Full VJP', "
              "sections 'What You Have' and 'Hard Constraints'; see make_two_key.py",
    "inputs": {
        "q": [[[1.0, 0.0, 0.0, 0.0]]],
        "k": [[[x, 0.0, 0.0, 0.0]], [[0.0, 0.0, 0.0, 0.0]]],
        "v": [[[1.0, 0.0, 0.0, 0.0]], [[0.0, 1.0, 0.0, 0.0]]],
        "dout": [[[g0, g1, 0.0, 0.0]]],
        "cu_q": [0, 1], "cu_k": [0, 2], "alibi_slopes": [[mu]],
        "softcap": c, "scale_multiplier": 0.75,
    },
    "expected": {
        "out": [[[p, 1.0 - p, 0.0, 0.0]]],
        "lse": [[math.log1p(math.exp(a0))]],
        "dq": [[[sigma * G * Tp * x, 0.0, 0.0, 0.0]]],
        "dk": [[[sigma * G * Tp, 0.0, 0.0, 0.0]], [[-sigma * G, 0.0, 0.0, 0.0]]],
        "dv": [[[p * g0, p * g1, 0.0, 0.0]], [[(1 - p) * g0, (1 - p) * g1, 0.0, 0.0]]],
    },
    "wrong_order_p": 1.0 / (1.0 + math.exp(-c * math.tanh((sigma * x - mu) / c))),
}
path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "two_key_worked_example.json")
with open(path, "w") as f:
    json.dump(case, f, indent=1)
    f.write("\n")
print("wrote", path)
