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

# VATP with its GQA union: Hq = 4 query heads over Hkv = 2 groups (G = 2, head h
# in group h // 2).  Token 0's value is (3, 4, 0, 0) in group 0 (l2 norm 5) and
# (5, 12, 0, 0) in group 1 (l2 norm 13); the heads' attention on it is
# 0.1, 0.2, 0.3, 0.4.  VATP = A * ||v|| = 0.5, 1.0, 3.9, 5.2 and the union takes
# the largest of each group: U = (1.0, 5.2).
add("vatp_norms_5_13_A_1234", {"vatp": [0.5, 1.0, 3.9, 5.2], "U": [1.0, 5.2]},
    "VATP[h] = A[h] * ||v_{h // 2}||_2 with norms 5 (3-4-5) and 13 (5-12-13); U = max per group",
    SELKV + " section 2, pipeline overview step 1 (VATP: attention times value norm) and"
    " step 2 (union over the query heads of a KV head)")

# Compensated decode: d = 4, scale 1/2, q = (2, 0, 0, 0) and two keys (10, 0, 0, 0)
# give the logit 10 twice; ln R = (0, ln 3) with alpha = 1 adds ln 3 to key 1.
# Normaliser e^10 + 3 e^10, so lse = 10 + ln 4 and o = v0/4 + 3 v1/4.
add("decode_lse_two_keys_bias_ln3", 10.0 + math.log(4.0),
    "logits 10 and 10 + ln 3: lse = ln(e^10 (1 + 3)) = 10 + ln 4",
    SELKV + " section 2, attention compensation (alpha * ln R added to the logit)")

# Rotary re-positioning with d = 4 (pairs (0, 2) and (1, 3)): pair i turns by
# delta * base^(-2i/d); pair 1 by delta * base^(-1/2).  base 10000, delta 7:
# 0.07 rad.
add("rope_d4_pair1_angle_base1e4_delta7", 7.0 * 10000.0 ** -0.5,
    "pair i = 1 of d = 4: angle = delta * base^(-2 * 1 / 4) = 7 / 100",
    SELKV + " section 2, pipeline overview step 6 (RoPE re-positioning); the"
    " frequency schedule base^(-2i/d) is the standard rotary one, the page gives none")

here = os.path.dirname(os.path.abspath(__file__))
with open(os.path.join(here, "closed_forms.json"), "w") as f:
    json.dump(forms, f, indent=1, sort_keys=True)
print(f"wrote {len(forms)} closed forms")
