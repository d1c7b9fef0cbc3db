"""The seeded input recipes (no GPU): deterministic per seed and set, distinct
across sets, with the shapes and distributions the recipes state."""

import numpy as np
import torch

from rmsnorm_activation_quantization_amd import inputs


def test_row_recipes_are_deterministic_and_rotate():
    a = inputs.row_inputs(inputs.FP8_TOKEN_SMALL)
    b = inputs.row_inputs(inputs.FP8_TOKEN_SMALL)
    c = inputs.row_inputs(inputs.FP8_TOKEN_SMALL, set_index=1)
    for k in ("x", "residual", "weight"):
        assert torch.equal(a[k], b[k]), f"{k} is not reproducible"
        assert a[k].dtype == torch.bfloat16
    assert not torch.equal(a["x"], c["x"]), "rotating sets must differ"
    assert a["x"].shape == (4, 2048) and a["weight"].shape == (2048,)


def test_row_distributions():
    d = inputs.row_inputs(inputs.DECODE_4096)
    x, w = d["x"].float(), d["weight"].float()
    assert abs(x.mean().item()) < 0.05 and abs(x.std().item() - 1.0) < 0.05
    assert abs(w.mean().item() - 1.0) < 0.02 and abs(w.std().item() - 0.1) < 0.02
    # fp16 rows are the same draws rounded to fp16
    d16 = inputs.row_inputs(inputs.DECODE_4096, dtype=torch.float16)
    assert torch.allclose(d16["x"].float(), x, rtol=1e-2, atol=1e-3)


def test_outliers_are_about_one_percent():
    d = inputs.row_inputs(inputs.FP8_GROUP_DECODE)
    plain = inputs.row_inputs(inputs.RowWorkload("no_outliers", 16, 4096, 1002))
    for k in ("x", "residual"):
        ratio = (d[k].float() / plain[k].float()).nan_to_num(1.0)
        frac = float((ratio.abs() > 10).float().mean())
        assert 0.005 < frac < 0.015, f"{k}: {frac:.4f} of elements are outliers"


def test_qk_recipe_and_strided_k():
    w = inputs.QK_DECODE
    d = inputs.qk_inputs(w)
    assert d["qg"].shape == (64, 2 * 16 * 256) and d["k"].shape == (64, 2 * 256) and d["q_w"].shape == (256,)
    assert abs(d["q_w"].float().std().item() - 0.1) < 0.02
    wide = inputs.qk_inputs(w, ld_k=1024)
    assert wide["k"].shape == (64, 1024)


def test_bits_round_trip():
    v = torch.randn(3, 5).to(torch.bfloat16)
    assert torch.equal(inputs.from_bits(inputs.bits(v)), v)
    h = torch.randn(3, 5).to(torch.float16)
    assert torch.equal(inputs.from_bits(inputs.bits(h), torch.float16), h)
    assert inputs.bits(v).dtype == np.uint16
