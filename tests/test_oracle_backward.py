"""Pins of the oracle's attention and RoPE gradients.

The pages train their models end to end (the 24 q / 8 KV model on page
"训练3.8B LLM至0.384 CORE，成本998美元 – Hugo Vergnes", section 设置), which
needs the gradients of causal GQA attention and of RoPE.  The pages print no
formula; the oracle writes the gradients of the plain definition out.  These
tests pin them to torch float64 autograd through scaled_dot_product_attention
(GQA by repeated KV heads) and through transformers' rotary helper, to central
finite differences, and to closed forms.
"""
import torch
import torch.nn.functional as F

import oracle
from rope_gqa_causal_amd import synth


def _inputs(B, S, Hq, Hkv, D, seed, dtype=torch.float32):
    g = synth.generator(seed)
    return (synth.normal((B, S, Hq, D), g, dtype), synth.normal((B, S, Hkv, D), g, dtype),
            synth.normal((B, S, Hkv, D), g, dtype), synth.normal((B, S, Hq, D), g, dtype))


def _autograd(q, k, v, dO):
    g = q.shape[2] // k.shape[2]
    qd, kd, vd = (t.to(torch.float64).transpose(1, 2).requires_grad_(True) for t in (q, k, v))
    o = F.scaled_dot_product_attention(qd, kd.repeat_interleave(g, dim=1), vd.repeat_interleave(g, dim=1),
                                       is_causal=True)
    o.backward(dO.to(torch.float64).transpose(1, 2))
    return [t.grad.transpose(1, 2) for t in (qd, kd, vd)]


def test_matches_torch_autograd_through_sdpa():
    for (B, S, Hq, Hkv, D, dt) in ((2, 13, 6, 2, 16, torch.float32), (1, 40, 4, 4, 32, torch.bfloat16),
                                   (1, 9, 8, 1, 8, torch.float32)):
        q, k, v, dO = _inputs(B, S, Hq, Hkv, D, S + Hq, dt)
        ours = oracle.attn_backward(q, k, v, dO)
        ref = _autograd(q, k, v, dO)
        for a, b, name in zip(ours, ref, ("dq", "dk", "dv")):
            assert torch.allclose(a, b, atol=1e-11, rtol=0), name


def test_central_finite_differences():
    # fp32 inputs (the oracle reads fp32 or bf16 exactly), a step of 2^-10
    # that is exact at these magnitudes, and the loss sum(o * dO) in fp64.
    B, S, Hq, Hkv, D = 1, 5, 2, 1, 4
    q, k, v, dO = _inputs(B, S, Hq, Hkv, D, 3)
    dq, dk, dv = oracle.attn_backward(q, k, v, dO)

    def loss(q_, k_, v_):
        return float((oracle.attn(q_, k_.transpose(1, 2), v_.transpose(1, 2)) * dO.to(torch.float64)).sum())

    h = 2.0 ** -10
    for t, grad, idx in ((q, dq, (0, 3, 1, 2)), (k, dk, (0, 1, 0, 3)), (v, dv, (0, 2, 0, 1)), (k, dk, (0, 4, 0, 0))):
        tp, tm = t.clone(), t.clone()
        tp[idx] += h
        tm[idx] -= h
        args_p = [tp if x is t else x for x in (q, k, v)]
        args_m = [tm if x is t else x for x in (q, k, v)]
        fd = (loss(*args_p) - loss(*args_m)) / (2 * h)
        assert abs(fd - grad[idx].item()) < 2e-5, (idx, fd, grad[idx].item())


def test_value_gradient_sums_and_gqa_is_summed_mha():
    B, S, Hq, Hkv, D = 2, 11, 4, 2, 8
    q, k, v, dO = _inputs(B, S, Hq, Hkv, D, 4)
    dq, dk, dv = oracle.attn_backward(q, k, v, dO)
    # Every weight row sums to one, so the value gradients of a group sum to
    # the group's output gradients.
    g = Hq // Hkv
    want = dO.to(torch.float64).view(B, S, Hkv, g, D).sum(dim=(1, 3))
    assert torch.allclose(dv.sum(dim=1), want, atol=1e-12, rtol=0)
    # GQA gradients = MHA gradients on repeated KV heads, summed per group.
    dq2, dk2, dv2 = oracle.attn_backward(q, k.repeat_interleave(g, dim=2), v.repeat_interleave(g, dim=2), dO)
    assert torch.allclose(dq, dq2, atol=1e-12, rtol=0)
    assert torch.allclose(dk, dk2.view(B, S, Hkv, g, D).sum(3), atol=1e-12, rtol=0)
    assert torch.allclose(dv, dv2.view(B, S, Hkv, g, D).sum(3), atol=1e-12, rtol=0)


def test_rope_gradient_is_the_inverse_rotation_and_matches_autograd():
    from transformers import LlamaConfig
    from transformers.models.llama.modeling_llama import LlamaRotaryEmbedding, apply_rotary_pos_emb

    B, S, H, D = 2, 5, 3, 32
    g = synth.normal((B, S, H, D), synth.generator(6), torch.float32)
    pos0 = torch.tensor([0, 700], dtype=torch.int32)
    ours = oracle.rope_grad_f64(g, pos0)
    # turning back what RoPE turned
    back = oracle.rope_grad_f64(oracle.rope_f64(g, pos0).to(torch.float32), pos0)
    assert torch.allclose(back, g.to(torch.float64), atol=1e-6, rtol=0)
    cfg = LlamaConfig(hidden_size=H * D, num_attention_heads=H, num_key_value_heads=H, head_dim=D,
                      rope_theta=10000.0, max_position_embeddings=4096)
    rot = LlamaRotaryEmbedding(cfg)
    pos = pos0[:, None].to(torch.int64) + torch.arange(S)[None, :]
    x = torch.zeros(B, H, S, D, dtype=torch.float64, requires_grad=True)
    cos, sin = rot(x, pos)
    y, _ = apply_rotary_pos_emb(x, x, cos, sin)
    y.backward(g.to(torch.float64).transpose(1, 2))
    # transformers forms the angle in float32: error ~ pos * 2^-24.
    assert torch.allclose(ours, x.grad.transpose(1, 2), atol=1e-4, rtol=0)
    for style in (oracle.ROPE_HALF, oracle.ROPE_INTERLEAVED):
        turned = oracle.rope_f64(g, pos0, 10000.0, style).to(torch.float32)
        inv = oracle.rope_grad_f64(turned, pos0, 10000.0, style)
        assert torch.allclose(inv, g.to(torch.float64), atol=1e-6, rtol=0)
