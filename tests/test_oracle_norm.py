"""Pins of the oracle's QK normalisation (RMS) before RoPE.

RMSNorm divides a vector by the root of the mean of its squares (page
"从零手训LLaMa：125M模型11小时训练全记录", core-architecture section); the 3.8B
model normalises q and k (page "训练3.8B LLM至0.384 CORE，成本998美元 – Hugo
Vergnes", section 设置).  The pages print no formula, epsilon or weight; the
reading here is eps = 1e-6 and no weight.  These tests pin the oracle to
torch's own rms_norm followed by transformers' LLaMA rotary helper, to closed
forms and to the invariances of the definition.
"""
import cmath
import math

import torch
import torch.nn.functional as F

import oracle
from rope_gqa_causal_amd import synth


def _x(shape, seed, dtype=torch.float32):
    return synth.normal(shape, synth.generator(seed), dtype)


def test_matches_torch_rms_norm_then_transformers_rotary():
    from transformers import LlamaConfig
    from transformers.models.llama.modeling_llama import LlamaRotaryEmbedding, apply_rotary_pos_emb

    B, S, H, D = 2, 6, 3, 64
    x = _x((B, S, H, D), 21)
    pos0 = torch.tensor([0, 90], dtype=torch.int32)
    ours = oracle.norm_rope_f64(x, pos0, 10000.0, oracle.ROPE_HALF, 1e-6)

    normed = F.rms_norm(x.to(torch.float64), (D,), eps=1e-6)
    cfg = LlamaConfig(hidden_size=H * D, num_attention_heads=H, num_key_value_heads=H,
                      head_dim=D, rope_theta=10000.0, max_position_embeddings=4096)
    rot = LlamaRotaryEmbedding(cfg)
    pos = (pos0[:, None].to(torch.int64) + torch.arange(S)[None, :])
    xt = normed.transpose(1, 2)
    cos, sin = rot(xt, pos)
    ref, _ = apply_rotary_pos_emb(xt, xt, cos, sin)
    # transformers forms the angle in float32: error ~ pos * 2^-24.
    assert torch.allclose(ours, ref.transpose(1, 2), atol=2e-5, rtol=0)


def test_position_zero_is_the_plain_rms_normalisation():
    x = _x((1, 1, 4, 32), 22)
    ours = oracle.norm_rope_f64(x, None, 10000.0, oracle.ROPE_HALF, 1e-6)
    xd = x.to(torch.float64)
    ref = xd / torch.sqrt(xd.pow(2).mean(-1, keepdim=True) + 1e-6)
    assert torch.allclose(ours, ref, atol=1e-14, rtol=0)


def test_without_eps_every_head_vector_has_unit_mean_square():
    x = _x((2, 5, 3, 128), 23, torch.bfloat16)
    pos0 = torch.tensor([7, 4000], dtype=torch.int32)
    for style in (oracle.ROPE_HALF, oracle.ROPE_INTERLEAVED):
        y = oracle.norm_rope_f64(x, pos0, 10000.0, style, 0.0)
        assert torch.allclose(y.pow(2).mean(-1), torch.ones(2, 5, 3, dtype=torch.float64), atol=1e-13, rtol=0)


def test_scale_invariance_and_eps_floor():
    x = _x((1, 3, 2, 64), 24)
    pos0 = torch.tensor([11], dtype=torch.int32)
    a = oracle.norm_rope_f64(x, pos0, 10000.0, oracle.ROPE_HALF, 0.0)
    b = oracle.norm_rope_f64(x * 4.0, pos0, 10000.0, oracle.ROPE_HALF, 0.0)  # exact scaling
    assert torch.allclose(a, b, atol=1e-14, rtol=0)
    # A vector far below eps is divided by sqrt(eps) instead: y ~ rope(x) / sqrt(eps).
    tiny = x * 2.0 ** -40
    y = oracle.norm_rope_f64(tiny, pos0, 10000.0, oracle.ROPE_HALF, 1e-6)
    r = oracle.rope_f64(tiny, pos0, 10000.0, oracle.ROPE_HALF) / math.sqrt(1e-6)
    assert torch.allclose(y, r, rtol=1e-9, atol=0)
    z = oracle.norm_rope_f64(torch.zeros(1, 1, 1, 16), None, 10000.0, oracle.ROPE_HALF, 1e-6)
    assert torch.equal(z, torch.zeros(1, 1, 1, 16, dtype=torch.float64))


def test_d2_is_normalised_complex_multiplication():
    x = torch.tensor([[[[3.0, -4.0]]]])  # mean square 12.5
    for pos in (0, 1, 5, 1000):
        y = oracle.norm_rope_f64(x, torch.tensor([pos], dtype=torch.int32), 10000.0, oracle.ROPE_HALF, 0.0)
        z = complex(3.0, -4.0) / math.sqrt(12.5) * cmath.exp(1j * pos)  # theta_0 = 1
        assert abs(y[0, 0, 0, 0].item() - z.real) < 1e-12 and abs(y[0, 0, 0, 1].item() - z.imag) < 1e-12
