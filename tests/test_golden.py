"""Hand-derived closed-form cases (tests/golden/closed_form_cases.json): the
oracle on the CPU and, under the gpu marker, the HIP path must reproduce
each expected bf16 pattern exactly."""
import json
import os

import numpy as np
import pytest
import torch

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
CASES = json.load(open(os.path.join(HERE, "golden", "closed_form_cases.json")))["cases"]


def build(case):
    Sq, Skv = case["Sq"], case["Skv"]
    fill = {"zeros": 0.0, "ones": 1.0}
    q = torch.full((1, 1, Sq, 128), fill[case["q"]], dtype=torch.float32)
    k = torch.full((1, 1, Skv, 128), fill[case["k"]], dtype=torch.float32)
    rows = np.array([case["v_rows"][j % len(case["v_rows"])] for j in range(Skv)], dtype=np.float32)
    v = torch.from_numpy(np.repeat(rows[:, None], 128, axis=1)[None, None].copy())
    return q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16)


def bits(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("case", CASES, ids=[c["name"] for c in CASES])
def test_oracle_reproduces_golden(case):
    q, k, v = build(case)
    res = oracle.attention(bits(q), bits(k), bits(v), layout="bhsd", scale=case["scale"], method=False)
    for mode, exp in case["expect"].items():
        assert np.all(res.rounded(mode) == int(exp, 16)), (mode, res.rounded(mode)[0, :4])


@pytest.mark.gpu
@pytest.mark.parametrize("case", CASES, ids=[c["name"] for c in CASES])
def test_hip_reproduces_golden(case):
    from bf16_attention_forward_amd import attn_fwd_bf16
    q, k, v = build(case)
    for mode, exp in case["expect"].items():
        o = attn_fwd_bf16(q.cuda(), k.cuda(), v.cuda(), layout="bhsd", scale=case["scale"], round_mode=mode)
        torch.cuda.synchronize()
        assert np.all(bits(o.cpu()) == int(exp, 16)), (mode, bits(o.cpu()).ravel()[:4])
