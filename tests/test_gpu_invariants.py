"""GPU-side invariants of the attention the pages define, each within the
bf16 bar, on seeded inputs:
  * V = 1 everywhere gives O = 1 (softmax rows sum to one) in prefill, in the
    split decode and in the one-workgroup decode walk;
  * shift invariance of RoPE scores (page "750美元从零训练3个LLM：一位开发者的
    实战复盘", section V1: the rotation makes q.k depend on the relative offset
    only): rotating every q and k at positions shifted by s leaves the
    attention output unchanged, for prefill and for decode;
  * a causal row never depends on later keys: changing every key and value
    after a row's slot leaves that row's output bitwise unchanged."""
import pytest
import torch

import rope_gqa_causal_amd as rgc
from rope_gqa_causal_amd import synth
from _util import assert_close

pytestmark = pytest.mark.gpu

ONE_BF16_ULP_BELOW_ONE = 2.0 ** -8


@pytest.mark.parametrize("D,Hq,Hkv,S", [(128, 24, 8, 700), (64, 12, 4, 333), (32, 4, 1, 129)])
def test_prefill_of_all_ones_values_is_one(D, Hq, Hkv, S):
    g = synth.generator(D + S)
    q = synth.normal((2, S, Hq, D), g).cuda()
    k = synth.normal((2, Hkv, S, D), g).cuda()
    v = torch.ones_like(k)
    o = rgc.gqa_attn_prefill(q, k, v)
    assert (o.float() - 1.0).abs().max().item() <= ONE_BF16_ULP_BELOW_ONE


@pytest.mark.parametrize("B,S_max", [(64, 2080), (2, 600)])  # split kernel; one-workgroup walk
def test_decode_of_all_ones_values_is_one(B, S_max):
    Hq, Hkv, D = 24, 8, 128
    g = synth.generator(B + S_max)
    q = synth.normal((B, Hq, D), g).cuda()
    k = synth.normal((B, Hkv, S_max, D), g).cuda()
    v = torch.ones_like(k)
    lens = synth.lengths(B, 1, S_max, g).cuda()
    o = rgc.gqa_attn_decode(q, k, v, lens, S_max)
    assert (o.float() - 1.0).abs().max().item() <= ONE_BF16_ULP_BELOW_ONE


def _rotated(x, shift):
    y = x.clone()
    rgc.rope_apply(y, torch.full((x.shape[0],), shift, dtype=torch.int32, device="cuda"))
    return y


@pytest.mark.parametrize("shift", [17, 12345])
def test_prefill_is_shift_invariant(shift):
    B, S, Hq, Hkv, D = 2, 400, 24, 8, 128
    g = synth.generator(shift)
    q, k, v = (t.cuda() for t in synth.qkv(B, S, Hq, Hkv, D, g))
    o0 = rgc.gqa_attn_prefill(_rotated(q, 0), _rotated(k, 0).transpose(1, 2), v.transpose(1, 2))
    o1 = rgc.gqa_attn_prefill(_rotated(q, shift), _rotated(k, shift).transpose(1, 2), v.transpose(1, 2))
    assert_close(o1, o0.cpu().double(), torch.bfloat16, f"prefill shifted by {shift}")


@pytest.mark.parametrize("B", [64, 2])  # split kernel; one-workgroup walk
def test_decode_is_shift_invariant(B):
    Hq, Hkv, D, S_max, shift = 24, 8, 128, 640, 4099
    g = synth.generator(B + 3)
    lens = synth.lengths(B, 1, S_max, g)
    k = synth.normal((B, S_max, Hkv, D), g).cuda()
    v = synth.normal((B, Hkv, S_max, D), g).cuda()
    q = synth.normal((B, 1, Hq, D), g).cuda()
    outs = []
    for s in (0, shift):
        kr = _rotated(k, s).transpose(1, 2).contiguous()  # key j at position s + j
        qr = q.clone()
        rgc.rope_apply(qr, (lens.cuda() - 1 + s).to(torch.int32))  # the query at s + L - 1
        outs.append(rgc.gqa_attn_decode(qr[:, 0], kr, v, lens.cuda(), S_max))
    assert_close(outs[1], outs[0].cpu().double(), torch.bfloat16, f"decode shifted by {shift}")


def test_prefill_rows_do_not_depend_on_later_keys():
    B, S, Hq, Hkv, D = 1, 512, 12, 4, 64
    g = synth.generator(8)
    q, k, v = (t.cuda() for t in synth.qkv(B, S, Hq, Hkv, D, g))
    kc, vc = k.transpose(1, 2).contiguous(), v.transpose(1, 2).contiguous()
    o = rgc.gqa_attn_prefill(q, kc, vc)
    cut = 300
    kc2, vc2 = kc.clone(), vc.clone()
    kc2[:, :, cut:] = synth.normal((B, Hkv, S - cut, D), g).cuda()
    vc2[:, :, cut:] = synth.normal((B, Hkv, S - cut, D), g).cuda()
    o2 = rgc.gqa_attn_prefill(q, kc2, vc2)
    assert torch.equal(o[:, :cut].cpu().view(torch.int16), o2[:, :cut].cpu().view(torch.int16))
