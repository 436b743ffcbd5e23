"""The attention comparison itself, on the CPU: it must accept the oracle's
own result rounded to bf16 (what an exact kernel would return) and reject a
result that drops one selected entry or mis-scales the scores."""
import numpy as np
import torch

from csa_synth import AttnWorkload, make_attn_inputs
from checker import attention_reference, compare_attention


def _round_bf16_bits(x):
    return torch.from_numpy(x).to(torch.float32).to(torch.bfloat16).view(torch.int16).numpy() \
        .view(np.uint16)


def _setup():
    aw = AttnWorkload("chk", B=1, S=200, T=50, H=32, D=64, n_sel=40)
    inp = make_attn_inputs(aw, seed=9, device="cpu")
    rows = np.arange(aw.S)
    return aw, inp, rows, attention_reference(inp, 0, rows, aw.softmax_scale)


def test_accepts_rounded_oracle():
    aw, inp, rows, (o, lse, a, dz) = _setup()
    compare_attention(_round_bf16_bits(o), lse.astype(np.float32), o, lse, a, dz)


def test_rejects_a_dropped_entry():
    aw, inp, rows, (o, lse, a, dz) = _setup()
    idx = inp["idx"].clone()
    idx[0, 150, 3] = -1                               # row 150 loses one entry
    o2, lse2, _, _ = attention_reference(dict(inp, idx=idx), 0, rows, aw.softmax_scale)
    try:
        compare_attention(_round_bf16_bits(o2), lse2.astype(np.float32), o, lse, a, dz)
    except AssertionError:
        return
    raise AssertionError("a dropped entry went unnoticed")


def test_rejects_wrong_scale():
    aw, inp, rows, (o, lse, a, dz) = _setup()
    o2, lse2, _, _ = attention_reference(inp, 0, rows, aw.softmax_scale * 1.01)
    try:
        compare_attention(_round_bf16_bits(o2), lse2.astype(np.float32), o, lse, a, dz)
    except AssertionError:
        return
    raise AssertionError("a 1% scale error went unnoticed")
