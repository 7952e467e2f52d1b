"""Writes closed_forms.json: values that follow from the pages' definitions by
hand derivation.  Uses only the standard library's ``math``; nothing here calls
the oracle or the GPU library.

Run:  python tests/golden/make_closed_forms.py
"""
import json
import math
import os

INFOKV = "[InfoKV] (aitrends.kr 68510)"
SELKV = "[SelKV] (gist.science 2607.16213)"

forms = {}


def add(name, value, derivation, cite):
    forms[name] = {"value": value, "derivation": derivation, "cite": cite}


for k in (64, 256):
    add(f"entropy_flat_k{k}", math.log(k),
        "k equal top logits: p = 1/k each, H = ln k",
        INFOKV + " Glossary, top-k restricted entropy; renormalised over the top k")
    # half the top k at x, half at x - ln 3: weights 3:1, p = 3/(2k) and 1/(2k)
    add(f"entropy_two_level_k{k}", math.log(2 * k) - 0.75 * math.log(3),
        "k/2 logits at x and k/2 at x - ln 3: H = (3/4) ln(2k/3) + (1/4) ln(2k)"
        " = ln(2k) - (3/4) ln 3",
        INFOKV + " Glossary, top-k restricted entropy")

tau = 1.0
add("distance_identical", tau, "cos = 1: D = 1 - 1 + tau", INFOKV + " Technical detail (tau)")
add("distance_opposite", 2.0 + tau, "cos = -1: D = 2 + tau", INFOKV + " Method")
add("distance_orthogonal", 1.0 + tau, "cos = 0: D = 1 + tau", INFOKV + " Method")

# Equal keys: every visible key gets the same logit, so window row r (position
# p_r = n - w + r) spreads 1/(p_r + 1) over keys 0..p_r.
n, w = 8, 4
A = []
for j in range(n):
    A.append(sum(1.0 / (n - w + r + 1) for r in range(w) if n - w + r >= j) / w)
add("window_attention_equal_keys_n8_w4", A,
    "A_j = (1/w) * sum over window rows r with p_r >= j of 1/(p_r + 1)",
    INFOKV + " Method, observation-window attention (causal, 1/sqrt(d) scale)")

# Adaptive budget: Ebar = [1, 2, 3], B = 100 -> x = [16.67, 33.33, 50]
add("adaptive_budget_123_B100", [17, 33, 50],
    "floor(x) = [16, 33, 50] sums to 99; the leftover 1 goes to layer 0",
    INFOKV + " Method / Glossary, adaptive budget allocation")
add("adaptive_budget_equal_L3_B10", [4, 3, 3],
    "x = 10/3 each, floor 3, leftover 1 to layer 0", INFOKV + " Method")

add("gate_orthogonal", 0.0, "cos = 0 -> g = 0", SELKV + " section 2, soft cosine gate")
add("gate_parallel", 1.0, "cos = 1 -> g = 1", SELKV + " section 2, soft cosine gate")
add("gate_antiparallel", 0.0, "cos = -1 -> g = max(-1, 0) = 0", SELKV + " section 2, soft cosine gate")

# One kept token t (A_t = a) with two parallel routed tokens (A = b, c):
# R = (a + b + c) / a.  a = 0.5, b = 0.25, c = 0.25 -> R = 2, ln R = ln 2.
add("ratio_two_parallel_routed", math.log(2.0),
    "R = (A_t + g1 A_1 + g2 A_2) / A_t with g = 1, A = (0.5, 0.25, 0.25)",
    SELKV + " section 2, attention compensation")

here = os.path.dirname(os.path.abspath(__file__))
with open(os.path.join(here, "closed_forms.json"), "w") as f:
    json.dump(forms, f, indent=1, sort_keys=True)
print(f"wrote {len(forms)} closed forms")
