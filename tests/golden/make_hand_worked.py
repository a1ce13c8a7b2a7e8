"""Writes hand_worked.json: one-token MoE layers whose routing and output follow
in closed form from the moe_ffn pseudocode of "Decoding Trillion-Parameter MoE
LLMs: Sparse Architecture and Agentic Intelligence" (section "Routing: Top-K
Experts Plus a Shared Expert") with the layer's readings (softmax or sigmoid
scores, selection-only bias, renormalised weights times a scale, SwiGLU experts).

Every expected number below is a closed form evaluated with `math`; nothing here
calls the oracle or the GPU library.

Shared construction: x = [1, 0]; expert e has W13[e] = [[ln 3, 0], [e + 1, 0]]
(gate row, up row) and W2[e] = [[1], [-2]], so g = ln 3, u = e + 1,
h_e = SiLU(ln 3) (e + 1) = (3/4) ln 3 (e + 1) and y_e = h_e * [1, -2].
"""
import json
import math
import os

L3 = math.log(3.0)


def experts(E):
    return ([[[L3, 0.0], [float(e + 1), 0.0]] for e in range(E)],
            [[[1.0], [-2.0]] for _ in range(E)])


def y(e):
    h = 0.75 * L3 * (e + 1)
    return [h, -2.0 * h]


def combo(ws, es):
    out = [0.0, 0.0]
    for w, e in zip(ws, es):
        ye = y(e)
        out = [out[0] + w * ye[0], out[1] + w * ye[1]]
    return [out]


cases = []
w13, w2 = experts(4)

# 1. softmax over logits ln1..ln4 = 0.1..0.4; top-2 = {2, 3}; renormalised 3/7, 4/7
cases.append(dict(
    name="softmax_top2_ln_logits", score="softmax", k=2, scale=1.0, bias=None,
    x=[[1.0, 0.0]], router=[[math.log(e + 1.0), 0.0] for e in range(4)], w13=w13, w2=w2,
    expect_topk_idx=[[2, 3]], expect_topk_w=[[3 / 7, 4 / 7]],
    expect_out=combo([3 / 7, 4 / 7], [2, 3]), atol=1e-6))

# 2. sigmoid scores 1/2, 3/4, 1/4, 3/4; bias [0, 0, 0.6, -0.1] -> keys .5 .75 .85 .65;
#    top-2 = {1, 2}; weights from the unbiased scores: 2.5 * (3/4, 1/4) = 1.875, 0.625
cases.append(dict(
    name="sigmoid_bias_selects_low_score_expert", score="sigmoid", k=2, scale=2.5,
    bias=[0.0, 0.0, 0.6, -0.1],
    x=[[1.0, 0.0]], router=[[0.0, 0.0], [L3, 0.0], [-L3, 0.0], [L3, 0.0]], w13=w13, w2=w2,
    expect_topk_idx=[[1, 2]], expect_topk_w=[[1.875, 0.625]],
    expect_out=combo([1.875, 0.625], [1, 2]), atol=1e-6))

# 3. all logits equal: ties go to the lower expert index; weights 1/2 each
cases.append(dict(
    name="all_tied_lowest_indices", score="softmax", k=2, scale=1.0, bias=None,
    x=[[1.0, 0.0]], router=[[0.0, 0.0]] * 4, w13=w13, w2=w2,
    expect_topk_idx=[[0, 1]], expect_topk_w=[[0.5, 0.5]],
    expect_out=combo([0.5, 0.5], [0, 1]), atol=1e-6))

doc = {
    "source": "closed forms from the moe_ffn pseudocode (Decoding Trillion-Parameter MoE LLMs, "
              "section 'Routing: Top-K Experts Plus a Shared Expert'); see make_hand_worked.py",
    "cases": cases,
}
with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "hand_worked.json"), "w") as f:
    json.dump(doc, f, indent=1)
