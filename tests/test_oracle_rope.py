"""Pins of the oracle's RoPE and bf16 rounding against things other than itself.

RoPE (page "750美元从零训练3个LLM：一位开发者的实战复盘", section V1; page
"从零手训LLaMa：125M模型11小时训练全记录", core-architecture section) is a
position-dependent rotation of q and k whose scores depend only on relative
distance.  The pages print no formula; these tests pin the oracle to
independent implementations (transformers' LLaMA and GPT-J rotary helpers),
to the complex-number form for D = 2, and to the properties the pages state.
"""
import cmath
import math

import pytest
import torch

import oracle
from rope_gqa_causal_amd import synth


def _x(shape, seed, dtype=torch.float32):
    return synth.normal(shape, synth.generator(seed), dtype)


def test_half_style_matches_transformers_llama():
    from transformers import LlamaConfig
    from transformers.models.llama.modeling_llama import LlamaRotaryEmbedding, apply_rotary_pos_emb

    B, S, H, D = 2, 9, 3, 32
    x = _x((B, S, H, D), 11)
    pos0 = torch.tensor([0, 37], dtype=torch.int32)
    ours = oracle.rope_f64(x, pos0, 10000.0, oracle.ROPE_HALF)

    cfg = LlamaConfig(hidden_size=H * D, num_attention_heads=H, num_key_value_heads=H,
                      head_dim=D, rope_theta=10000.0, max_position_embeddings=4096)
    rot = LlamaRotaryEmbedding(cfg)
    pos = (pos0[:, None].to(torch.int64) + torch.arange(S)[None, :])
    xt = x.to(torch.float64).transpose(1, 2)            # [B,H,S,D]
    cos, sin = rot(xt, pos)
    ref, _ = apply_rotary_pos_emb(xt, xt, cos, sin)
    ref = ref.transpose(1, 2)
    # transformers forms the angle in float32: error ~ pos * 2^-24.
    assert torch.allclose(ours, ref, atol=2e-5, rtol=0)


def test_interleaved_style_matches_transformers_gptj():
    from transformers.models.gptj.modeling_gptj import apply_rotary_pos_emb, create_sinusoidal_positions

    B, S, H, D = 2, 7, 2, 16
    x = _x((B, S, H, D), 12)
    pos0 = torch.tensor([3, 50], dtype=torch.int32)
    ours = oracle.rope_f64(x, pos0, 10000.0, oracle.ROPE_INTERLEAVED)

    table = create_sinusoidal_positions(128, D)               # [pos, D]: sin | cos
    pos = (pos0[:, None].to(torch.int64) + torch.arange(S)[None, :])
    sincos = table[pos].to(torch.float64)                     # [B,S,D]
    sin, cos = torch.split(sincos, D // 2, dim=-1)
    ref = apply_rotary_pos_emb(x.to(torch.float64), sin, cos)
    assert torch.allclose(ours, ref, atol=2e-5, rtol=0)


@pytest.mark.parametrize("pos", [0, 1, 5, 1000, 123456])
def test_d2_is_complex_multiplication(pos):
    # D = 2: theta_0 = base^0 = 1, so RoPE multiplies a + ib by e^{i*pos}.
    x = _x((1, 1, 1, 2), 13 + pos)
    out = oracle.rope_f64(x, torch.tensor([pos], dtype=torch.int32), 10000.0, oracle.ROPE_HALF)
    z = complex(float(x[0, 0, 0, 0]), float(x[0, 0, 0, 1])) * cmath.exp(1j * pos)
    assert abs(out[0, 0, 0, 0].item() - z.real) < 1e-12
    assert abs(out[0, 0, 0, 1].item() - z.imag) < 1e-12


@pytest.mark.parametrize("D,base", [(8, 10000.0), (64, 10000.0), (128, 500000.0)])
def test_frequencies_form_the_geometric_ladder(D, base):
    # Rotating the unit vector on the first coordinate of pair i by one
    # position reveals the pair's angle theta_i.  The ladder starts at 1 rad,
    # shrinks by base^(-2/D) per pair, and one step past the end reaches 1/base.
    half = D // 2
    x = torch.zeros((1, 1, half, D), dtype=torch.float32)
    for i in range(half):
        x[0, 0, i, i] = 1.0
    out = oracle.rope_f64(x, torch.tensor([1], dtype=torch.int32), base, oracle.ROPE_HALF)
    th = [math.atan2(out[0, 0, i, i + half].item(), out[0, 0, i, i].item()) for i in range(half)]
    assert abs(th[0] - 1.0) < 1e-12
    r = base ** (-2.0 / D)
    for i in range(1, half):
        assert abs(th[i] / th[i - 1] - r) < 1e-9
    assert abs(th[-1] * r - 1.0 / base) < 1e-12 / base


def test_norm_of_every_pair_is_preserved_and_position_zero_is_identity():
    B, S, H, D = 1, 6, 2, 32
    x = _x((B, S, H, D), 14)
    out = oracle.rope_f64(x, torch.tensor([17], dtype=torch.int32), 10000.0, oracle.ROPE_HALF)
    xd = x.to(torch.float64)
    n_in = xd[..., :D // 2] ** 2 + xd[..., D // 2:] ** 2
    n_out = out[..., :D // 2] ** 2 + out[..., D // 2:] ** 2
    assert torch.allclose(n_in, n_out, atol=1e-12, rtol=1e-12)
    ident = oracle.rope_f64(x[:, :1], torch.tensor([0], dtype=torch.int32), 10000.0, oracle.ROPE_HALF)
    assert torch.equal(ident, xd[:, :1])


@pytest.mark.parametrize("style", [oracle.ROPE_HALF, oracle.ROPE_INTERLEAVED])
def test_scores_depend_only_on_relative_offset(style):
    # The property the V1 section of the first page states for RoPE.
    D = 64
    q = _x((1, 1, 1, D), 15)
    k = _x((1, 1, 1, D), 16)
    for m, n, s in [(3, 11, 100), (40, 2, 7), (0, 0, 999), (1500, 1499, 3000)]:
        def score(a, b):
            qa = oracle.rope_f64(q, torch.tensor([a], dtype=torch.int32), 10000.0, style)
            kb = oracle.rope_f64(k, torch.tensor([b], dtype=torch.int32), 10000.0, style)
            return float((qa * kb).sum())
        s0, s1 = score(m, n), score(m + s, n + s)
        assert abs(s0 - s1) <= 1e-11 * max(1.0, abs(s0))


def test_interleaved_is_a_fixed_permutation_of_half():
    # interleaved(x) = P^T half(P x) where P moves x_{2i} -> i, x_{2i+1} -> i + D/2.
    D = 16
    x = _x((2, 3, 2, D), 17)
    perm = torch.tensor([2 * i for i in range(D // 2)] + [2 * i + 1 for i in range(D // 2)])
    inv = torch.argsort(perm)
    pos0 = torch.tensor([5, 900], dtype=torch.int32)
    inter = oracle.rope_f64(x, pos0, 10000.0, oracle.ROPE_INTERLEAVED)
    half = oracle.rope_f64(x[..., perm].contiguous(), pos0, 10000.0, oracle.ROPE_HALF)
    assert torch.allclose(inter, half[..., inv], atol=1e-13, rtol=0)


def test_v_is_not_touched_and_in_place_rounds_once():
    x = _x((1, 4, 2, 32), 18, torch.bfloat16)
    exact = oracle.rope_f64(x, torch.tensor([300], dtype=torch.int32), 10000.0, oracle.ROPE_HALF)
    y = x.clone()
    oracle.rope_apply_(y, torch.tensor([300], dtype=torch.int32), 10000.0, oracle.ROPE_HALF)
    assert torch.equal(y, oracle.round_to_bf16(exact))


def test_bf16_rounding_matches_torch_bit_for_bit():
    # torch's float32 -> bfloat16 cast is round-to-nearest-even: a library pin
    # for the oracle's rounding on every float32 input kind.
    g = synth.generator(19)
    vals = torch.randn(4000, generator=g, dtype=torch.float32) * torch.exp2(
        torch.randint(-140, 128, (4000,), generator=g).float())
    bits = torch.randint(0, 2 ** 16, (2000,), generator=g, dtype=torch.int32)
    ties = ((bits << 16) | 0x8000).view(torch.float32)      # exact halfway cases
    special = torch.tensor([0.0, -0.0, float("inf"), -float("inf"), 3.4028234e38,
                            -3.4e38, 1e-45, -1e-45, 1.1754944e-38, 9.2e-41], dtype=torch.float32)
    x = torch.cat([vals, ties, special])
    x = x[torch.isfinite(x) | torch.isinf(x)]
    want = x.to(torch.bfloat16).view(torch.int16).to(torch.int32) & 0xFFFF
    got = torch.tensor([oracle.bf16_bits(float(v)) for v in x.tolist()], dtype=torch.int32)
    assert torch.equal(got, want)
