"""GPU parity: RoPE and cache append against the fp64 oracle."""
import pytest
import torch

import oracle
import rope_gqa_causal_amd as rgc
from rope_gqa_causal_amd import synth
from _util import assert_close

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("style", [rgc.ROPE_HALF, rgc.ROPE_INTERLEAVED])
@pytest.mark.parametrize("D", [2, 6, 32, 64, 128])
def test_rope_fp32(style, D):
    B, S, H = 3, 37, 5
    x = synth.normal((B, S, H, D), synth.generator(D + style), torch.float32)
    pos0 = torch.tensor([0, 4093, 123457], dtype=torch.int32)
    ref = oracle.rope_f64(x, pos0, 10000.0, style)
    y = x.cuda()
    rgc.rope_apply(y, pos0.cuda(), 10000.0, style)
    assert_close(y, ref, torch.float32, f"rope fp32 D={D} style={style}")


@pytest.mark.parametrize("style", [rgc.ROPE_HALF, rgc.ROPE_INTERLEAVED])
@pytest.mark.parametrize("D", [64, 128])
def test_rope_bf16(style, D):
    B, S, H = 2, 129, 8
    x = synth.normal((B, S, H, D), synth.generator(100 + D), torch.bfloat16)
    pos0 = torch.tensor([0, 1919], dtype=torch.int32)
    exact = oracle.rope_f64(x, pos0, 10000.0, style)
    once = oracle.rope_apply_(x.clone(), pos0, 10000.0, style)
    y = x.cuda()
    rgc.rope_apply(y, pos0.cuda(), 10000.0, style)
    assert_close(y, exact, torch.bfloat16, "rope bf16")
    # The GPU rounds an fp32 result once; it may differ from the single
    # rounding of the exact value only where fp32 error straddles a tie.
    same = (y.cpu().view(torch.int16) == once.view(torch.int16)).float().mean().item()
    assert same > 0.99


def test_rope_strided_heads_and_no_position_array():
    # q as a view into a packed [B,S,3,H,D] qkv buffer; pos0 = NULL means 0.
    B, S, H, D = 2, 16, 4, 64
    qkv = synth.normal((B, S, 3, H, D), synth.generator(7), torch.bfloat16)
    q = qkv[:, :, 0]
    ref = oracle.rope_f64(q, None, 10000.0, rgc.ROPE_HALF)
    g = qkv.cuda()
    rgc.rope_apply(g[:, :, 0], None)
    assert_close(g[:, :, 0], ref, torch.bfloat16, "strided rope")
    assert torch.equal(g[:, :, 1:].cpu(), qkv[:, :, 1:])  # k and v untouched


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("D", [32, 64, 128])
def test_append_bit_exact(dtype, D):
    B, Hkv, S_max, S_new = 4, 3, 40, 7
    g = synth.generator(D)
    kc, vc = synth.nan_cache(B, Hkv, S_max, D, dtype)
    k_new = synth.normal((B, S_new, Hkv, D), g, dtype)
    v_new = synth.normal((B, S_new, Hkv, D), g, dtype)
    pos0 = torch.tensor([0, 5, 33, 17], dtype=torch.int32)
    kref, vref = kc.clone(), vc.clone()
    assert oracle.kv_cache_append_(kref, vref, k_new, v_new, pos0) == 0
    kg, vg = kc.cuda(), vc.cuda()
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    rgc.kv_cache_append(kg, vg, k_new.cuda(), v_new.cuda(), pos0.cuda(), err)
    ibits = torch.int16 if dtype == torch.bfloat16 else torch.int32
    assert torch.equal(kg.cpu().view(ibits), kref.view(ibits))
    assert torch.equal(vg.cpu().view(ibits), vref.view(ibits))
    assert err.item() == 0


def test_append_out_of_capacity_is_flagged_and_skipped():
    B, Hkv, S_max, D, S_new = 2, 2, 16, 64, 4
    g = synth.generator(3)
    kc, vc = synth.nan_cache(B, Hkv, S_max, D)
    k_new = synth.normal((B, S_new, Hkv, D), g)
    pos0 = torch.tensor([2, 14], dtype=torch.int32)   # second sequence overflows by 2
    kref, vref = kc.clone(), vc.clone()
    oracle.kv_cache_append_(kref, vref, k_new, k_new, pos0)
    kg, vg = kc.cuda(), vc.cuda()
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    rgc.kv_cache_append(kg, vg, k_new.cuda(), k_new.cuda(), pos0.cuda(), err)
    assert err.item() == 1
    assert torch.equal(kg.cpu().view(torch.int16), kref.view(torch.int16))


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("style", [rgc.ROPE_HALF, rgc.ROPE_INTERLEAVED])
@pytest.mark.parametrize("S,D", [(1, 128), (37, 64), (5, 32)])
def test_rope_append_equals_rope_then_append_bit_for_bit(dtype, style, S, D):
    B, Hq, Hkv, S_max = 3, 6, 2, 64
    g = synth.generator(S * D + style)
    q, k, v = synth.qkv(B, S, Hq, Hkv, D, g, dtype)
    pos0 = torch.tensor([0, 9, S_max - S], dtype=torch.int32).cuda()
    # separate calls
    q1, k1 = q.cuda(), k.cuda().clone()
    kc1, vc1 = [t.cuda() for t in synth.nan_cache(B, Hkv, S_max, D, dtype)]
    rgc.rope_apply(q1, pos0, 10000.0, style)
    rgc.rope_apply(k1, pos0, 10000.0, style)
    rgc.kv_cache_append(kc1, vc1, k1, v.cuda(), pos0)
    # fused
    q2, k2 = q.cuda(), k.cuda()
    kc2, vc2 = [t.cuda() for t in synth.nan_cache(B, Hkv, S_max, D, dtype)]
    rgc.rope_append(q2, k2, v.cuda(), kc2, vc2, pos0, 10000.0, style)
    ibits = torch.int16 if dtype == torch.bfloat16 else torch.int32
    assert torch.equal(q1.cpu().view(ibits), q2.cpu().view(ibits))
    assert torch.equal(kc1.cpu().view(ibits), kc2.cpu().view(ibits))
    assert torch.equal(vc1.cpu().view(ibits), vc2.cpu().view(ibits))
    assert torch.equal(k2.cpu().view(ibits), k.view(ibits))  # k_new itself is not rotated


def test_rope_append_matches_the_oracle_and_flags_capacity():
    B, S, Hq, Hkv, D, S_max = 2, 4, 12, 4, 64, 40
    g = synth.generator(77)
    q, k, v = synth.qkv(B, S, Hq, Hkv, D, g)
    pos0 = torch.tensor([3, 38], dtype=torch.int32)   # second sequence runs 2 slots past the end
    ref_q = oracle.rope_f64(q, pos0)
    ref_k = oracle.rope_apply_(k.clone(), pos0)
    kc_ref, vc_ref = synth.nan_cache(B, Hkv, S_max, D)
    oracle.kv_cache_append_(kc_ref, vc_ref, ref_k, v, pos0)
    qg = q.cuda()
    kc, vc = [t.cuda() for t in synth.nan_cache(B, Hkv, S_max, D)]
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    rgc.rope_append(qg, k.cuda(), v.cuda(), kc, vc, pos0.cuda(), err_flag=err)
    assert err.item() == 1
    assert_close(qg, ref_q, torch.bfloat16, "fused rope q")
    assert torch.equal(vc.cpu().view(torch.int16), vc_ref.view(torch.int16))
    got, want = kc.cpu(), kc_ref
    written = ~torch.isnan(want)
    assert torch.equal(torch.isnan(got), torch.isnan(want))          # same slots written
    assert (got[written].double() - want[written].double()).abs().max().item() <= 2 ** -7 * 4


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("style", [rgc.ROPE_HALF, rgc.ROPE_INTERLEAVED])
@pytest.mark.parametrize("S,D", [(1, 128), (19, 64), (5, 32)])
def test_norm_rope_append_matches_the_oracle(dtype, style, S, D):
    B, Hq, Hkv, S_max, eps = 3, 6, 2, 64, 1e-6
    g = synth.generator(300 + S * D + style)
    q, k, v = synth.qkv(B, S, Hq, Hkv, D, g, dtype)
    q = q * 3.0  # away from unit scale, so the normalisation matters
    pos0 = torch.tensor([0, 17, S_max - S], dtype=torch.int32)
    ref_q = oracle.norm_rope_f64(q, pos0, 10000.0, style, eps)
    ref_k = oracle.norm_rope_f64(k, pos0, 10000.0, style, eps)
    qg = q.cuda()
    kc, vc = [t.cuda() for t in synth.nan_cache(B, Hkv, S_max, D, dtype)]
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    rgc.norm_rope_append(qg, k.cuda(), v.cuda(), kc, vc, pos0.cuda(), 10000.0, style, eps, err_flag=err)
    assert err.item() == 0
    assert_close(qg, ref_q, dtype, "normalised rope q")
    ibits = torch.int16 if dtype == torch.bfloat16 else torch.int32
    kc, vc = kc.cpu(), vc.cpu()
    for b in range(B):
        sl = slice(int(pos0[b]), int(pos0[b]) + S)
        assert_close(kc[b, :, sl].transpose(0, 1), ref_k[b], dtype, "normalised rope k in cache")
        assert torch.equal(vc[b, :, sl].transpose(0, 1).contiguous().view(ibits), v[b].contiguous().view(ibits))
    outside = torch.ones(S_max, dtype=torch.bool)
    for b in range(B):
        m = outside.clone()
        m[int(pos0[b]):int(pos0[b]) + S] = False
        assert torch.isnan(kc[b, :, m].float()).all() and torch.isnan(vc[b, :, m].float()).all()


def test_norm_rope_append_of_zero_rows_is_zero_and_plain_prologue_is_unchanged():
    B, S, Hq, Hkv, D, S_max = 2, 3, 4, 2, 64, 16
    z = torch.zeros(B, S, Hq, D, dtype=torch.bfloat16, device="cuda")
    zk = torch.zeros(B, S, Hkv, D, dtype=torch.bfloat16, device="cuda")
    kc = torch.full((B, Hkv, S_max, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    vc = kc.clone()
    pos0 = torch.tensor([0, 5], dtype=torch.int32, device="cuda")
    rgc.norm_rope_append(z, zk, zk, kc, vc, pos0, eps=1e-6)
    assert torch.equal(z, torch.zeros_like(z))
    assert torch.equal(kc[0, :, :S], torch.zeros(Hkv, S, D, dtype=torch.bfloat16, device="cuda"))
