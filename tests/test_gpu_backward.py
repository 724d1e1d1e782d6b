"""GPU parity: gradients of causal GQA self-attention and of RoPE against the fp64 oracle."""
import pytest
import torch

import oracle
import rope_gqa_causal_amd as rgc
from rope_gqa_causal_amd import synth
from _util import assert_close, assert_close_grad

pytestmark = pytest.mark.gpu


def _forward(B, S, Hq, Hkv, D, seed):
    g = synth.generator(seed)
    q, k, v = synth.qkv(B, S, Hq, Hkv, D, g)
    d_o = synth.normal((B, S, Hq, D), g)
    qg, kg, vg = q.cuda(), k.cuda(), v.cuda()
    lse = torch.empty((B, Hq, S), dtype=torch.float32, device="cuda")
    o = rgc.gqa_attn_prefill(qg, kg.transpose(1, 2), vg.transpose(1, 2), lse=lse)
    return q, k, v, d_o, qg, kg, vg, o, lse


BACKWARD_CASES = [
    # B, S, Hq, Hkv, D
    (2, 100, 6, 2, 64),     # g = 3, ragged tails of every block
    (1, 300, 4, 4, 128),    # g = 1
    (2, 77, 8, 1, 32),      # MQA, D 32
    (1, 161, 24, 8, 128),   # the 3.8B head layout
    (1, 1, 2, 1, 64),       # a single row
    # dQ's pipelined loop: several unmasked steps with a previous tile, the
    # diagonal tile and the tail, and a ragged last key tile (1000 = 15 x 64 + 40)
    (1, 1000, 4, 2, 128),
    (1, 640, 2, 1, 64),     # whole 64-key tiles only (no ragged tile), D 64
    (1, 129, 2, 2, 32),     # one row past a 128-row block, D 32
]


@pytest.mark.parametrize("case", BACKWARD_CASES, ids=lambda c: f"B{c[0]}S{c[1]}H{c[2]}/{c[3]}D{c[4]}")
def test_attention_backward_bf16(case):
    B, S, Hq, Hkv, D = case
    q, k, v, d_o, qg, kg, vg, o, lse = _forward(B, S, Hq, Hkv, D, S + D)
    dq, dk, dv = rgc.gqa_attn_backward(qg, kg, vg, o, d_o.cuda(), lse)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.attn_backward(q, k, v, d_o)
    assert_close_grad(dv, rv, "dv")
    assert_close_grad(dk, rk, "dk")
    assert_close_grad(dq, rq, "dq")


def test_backward_on_the_3p8b_layout_sampled():
    # 3.8B heads (24 q / 8 KV, D 128) at 1024 tokens, batch 2, launched as a
    # training step would; the oracle's full backward runs on the first
    # sequence (it is exact per sequence).
    B, S, Hq, Hkv, D = 2, 1024, 24, 8, 128
    q, k, v, d_o, qg, kg, vg, o, lse = _forward(B, S, Hq, Hkv, D, 77)
    dq, dk, dv = rgc.gqa_attn_backward(qg, kg, vg, o, d_o.cuda(), lse)
    rq, rk, rv = oracle.attn_backward(q[:1], k[:1], v[:1], d_o[:1])
    assert_close_grad(dv[:1], rv, "dv")
    assert_close_grad(dk[:1], rk, "dk")
    assert_close_grad(dq[:1], rq, "dq")


def test_backward_at_the_bench_shape_sampled():
    # The batch the bench times (8 x 2048 tokens, 24 q / 8 KV, D 128), in
    # that launch configuration; the oracle's exact backward runs on one
    # sequence (the gradients of different sequences are independent).
    B, S, Hq, Hkv, D = 8, 2048, 24, 8, 128
    q, k, v, d_o, qg, kg, vg, o, lse = _forward(B, S, Hq, Hkv, D, 303)
    dq, dk, dv = rgc.gqa_attn_backward(qg, kg, vg, o, d_o.cuda(), lse)
    b = 5
    rq, rk, rv = oracle.attn_backward(q[b:b + 1], k[b:b + 1], v[b:b + 1], d_o[b:b + 1])
    assert_close_grad(dv[b:b + 1], rv, "dv")
    assert_close_grad(dk[b:b + 1], rk, "dk")
    assert_close_grad(dq[b:b + 1], rq, "dq")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("style", [rgc.ROPE_HALF, rgc.ROPE_INTERLEAVED])
def test_rope_backward_matches_the_oracle_and_undoes_the_rotation(dtype, style):
    B, S, H, D = 2, 33, 5, 64
    g = synth.normal((B, S, H, D), synth.generator(12 + style), dtype)
    pos0 = torch.tensor([0, 3000], dtype=torch.int32)
    ref = oracle.rope_grad_f64(g, pos0, 10000.0, style)
    gg = g.cuda()
    rgc.rope_backward(gg, pos0.cuda(), 10000.0, style)
    assert_close(gg, ref, dtype, "rope gradient")
    if dtype == torch.float32:
        x = g.cuda()
        rgc.rope_apply(x, pos0.cuda(), 10000.0, style)
        rgc.rope_backward(x, pos0.cuda(), 10000.0, style)
        assert (x.cpu() - g).abs().max().item() < 1e-5
