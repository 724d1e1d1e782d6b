"""GPU parity: the one-launch generation step (gqa_attn_decode_rope_append)
against the two-launch step (rope_append, then gqa_attn_decode) bit for bit,
and against the fp64 oracle."""
import pytest
import torch

import oracle
import rope_gqa_causal_amd as rgc
from rope_gqa_causal_amd import synth
from _util import assert_close

pytestmark = pytest.mark.gpu

I16 = torch.int16


def _inputs(B, Hq, Hkv, D, S_max, lens, seed):
    """Random caches whose new slots (lens - 1) hold NaN, so a read of a slot
    the step is meant to fill shows up in the output; fresh q, k_new, v_new."""
    g = synth.generator(seed)
    kc, vc = synth.filled_cache(B, Hkv, S_max, D, g)
    for b, L in enumerate(lens.tolist()):
        if 1 <= L <= S_max:
            kc[b, :, L - 1] = float("nan")
            vc[b, :, L - 1] = float("nan")
    q = synth.normal((B, Hq, D), g)
    k_new = synth.normal((B, Hkv, D), g)
    v_new = synth.normal((B, Hkv, D), g)
    return q, k_new, v_new, kc, vc


def _two_launch(q, k_new, v_new, kc, vc, lens, max_len, style, lse):
    qr = q.clone()
    rgc.rope_append(qr[:, None], k_new[:, None], v_new[:, None], kc, vc, lens - 1, 10000.0, style)
    return rgc.gqa_attn_decode(qr, kc, vc, lens, max_len, lse=lse)


@pytest.mark.parametrize("style", [rgc.ROPE_HALF, rgc.ROPE_INTERLEAVED])
@pytest.mark.parametrize("D", [32, 64, 128])
@pytest.mark.parametrize("group", [1, 3, 8])
def test_fused_step_equals_prologue_then_decode_bit_for_bit(style, D, group):
    Hkv = 2
    Hq = Hkv * group
    S_max = 700
    # One key, chunk edges for either chunk length (128 / 256 / 512 keys),
    # and long ones.
    lens = torch.tensor([1, 2, 128, 129, 256, 257, 512, 513, 699, 700], dtype=torch.int32)
    B = lens.numel()
    q, k_new, v_new, kc, vc = _inputs(B, Hq, Hkv, D, S_max, lens, seed=D * 10 + group + style)
    dev = [t.cuda() for t in (q, k_new, v_new, kc, vc)]
    q_a, kn_a, vn_a, kc_a, vc_a = [t.clone() for t in dev]
    q_b, kn_b, vn_b, kc_b, vc_b = [t.clone() for t in dev]
    lens_g = lens.cuda()
    lse_a = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    lse_b = torch.empty_like(lse_a)
    o_a = _two_launch(q_a, kn_a, vn_a, kc_a, vc_a, lens_g, S_max, style, lse_a)
    o_b = rgc.gqa_attn_decode_rope_append(q_b, kn_b, vn_b, kc_b, vc_b, lens_g, S_max, style=style, lse=lse_b)
    assert torch.isfinite(o_b.float()).all(), "the fused step read a slot it was to fill"
    assert torch.equal(o_a.cpu().view(I16), o_b.cpu().view(I16))
    assert torch.equal(lse_a.cpu(), lse_b.cpu())
    assert torch.equal(kc_a.cpu().view(I16), kc_b.cpu().view(I16))
    assert torch.equal(vc_a.cpu().view(I16), vc_b.cpu().view(I16))
    assert torch.equal(q_b.cpu().view(I16), q.view(I16))  # q is left unrotated
    assert torch.equal(kn_b.cpu().view(I16), k_new.view(I16))


@pytest.mark.parametrize("style", [rgc.ROPE_HALF, rgc.ROPE_INTERLEAVED])
def test_fused_step_matches_the_oracle(style):
    B, Hq, Hkv, D, S_max = 6, 12, 4, 64, 400
    lens = torch.tensor([1, 63, 64, 200, 399, 400], dtype=torch.int32)
    q, k_new, v_new, kc, vc = _inputs(B, Hq, Hkv, D, S_max, lens, seed=500 + style)
    # The oracle's step: RoPE at position lens - 1 (rounded to bf16 as the
    # stored q and k are), append, attend.
    pos = lens - 1
    q_r = oracle.rope_apply_(q[:, None].clone(), pos, 10000.0, style)[:, 0]
    k_r = oracle.rope_apply_(k_new[:, None].clone(), pos, 10000.0, style)
    kc_ref, vc_ref = kc.clone(), vc.clone()
    assert oracle.kv_cache_append_(kc_ref, vc_ref, k_r, v_new[:, None], pos) == 0
    ref, ref_lse = oracle.attn_decode(q_r, kc_ref, vc_ref, lens, want_lse=True)
    kg, vg = kc.cuda(), vc.cuda()
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    o = rgc.gqa_attn_decode_rope_append(q.cuda(), k_new.cuda(), v_new.cuda(), kg, vg, lens.cuda(), S_max,
                                        style=style, lse=lse)
    assert_close(o, ref, torch.bfloat16, f"fused step style={style}")
    assert (lse.cpu().double() - ref_lse).abs().max().item() <= 1e-3
    assert torch.equal(vg.cpu().view(I16), vc_ref.view(I16))
    # The rotated k is one fp32 rotation rounded once; the oracle rounds the
    # exact rotation: they may differ by one bf16 ulp at a rounding tie.
    got, want = kg.cpu().double(), kc_ref.double()
    assert (got - want).abs().max().item() <= 2.0 ** -7 * 4


def test_fused_step_flags_a_bad_length_and_leaves_its_cache():
    B, Hq, Hkv, D, S_max, max_len = 3, 6, 2, 128, 300, 256
    lens = torch.tensor([10, 0, 257], dtype=torch.int32)   # 0 and 257 > max_len are invalid
    q, k_new, v_new, kc, vc = _inputs(B, Hq, Hkv, D, S_max, lens, seed=9)
    kg, vg = kc.cuda(), vc.cuda()
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    o = rgc.gqa_attn_decode_rope_append(q.cuda(), k_new.cuda(), v_new.cuda(), kg, vg, lens.cuda(), max_len,
                                        err_flag=err).cpu()
    assert err.item() == 1
    assert torch.isnan(o[1].float()).all() and torch.isnan(o[2].float()).all()
    assert torch.isfinite(o[0].float()).all()
    # the invalid sequences' caches are untouched (NaN canaries included)
    for b in (1, 2):
        assert torch.equal(kg[b].cpu().view(I16), kc[b].view(I16))
        assert torch.equal(vg[b].cpu().view(I16), vc[b].view(I16))


def test_fused_step_on_the_ragged_decode_workload():
    w = synth.WORKLOADS["ragged_decode"]
    g = synth.generator(w.seed)
    lens0 = synth.lengths(w.B, w.len_lo, w.len_hi, g)
    S_max = w.len_hi + w.steps
    kc, vc = synth.filled_cache(w.B, w.Hkv, S_max, w.D, g, w.dtype)
    q = synth.normal((w.B, w.Hq, w.D), g, w.dtype)
    k_new = synth.normal((w.B, w.Hkv, w.D), g, w.dtype)
    v_new = synth.normal((w.B, w.Hkv, w.D), g, w.dtype)
    lens = lens0 + 1
    ws = rgc.decode_workspace(w.B, w.Hq, w.Hkv, w.D, S_max)
    kc_a, vc_a, kc_b, vc_b = kc.cuda(), vc.cuda(), kc.cuda(), vc.cuda()
    o_a = _two_launch(q.cuda(), k_new.cuda(), v_new.cuda(), kc_a, vc_a, lens.cuda(), S_max, rgc.ROPE_HALF, None)
    o_b = rgc.gqa_attn_decode_rope_append(q.cuda(), k_new.cuda(), v_new.cuda(), kc_b, vc_b, lens.cuda(), S_max, ws)
    assert torch.equal(o_a.cpu().view(I16), o_b.cpu().view(I16))
    assert torch.equal(kc_a.cpu().view(I16), kc_b.cpu().view(I16))
    assert torch.equal(vc_a.cpu().view(I16), vc_b.cpu().view(I16))
    o_b = o_b.cpu()
    q_r = oracle.rope_apply_(q[:, None].clone(), lens - 1)[:, 0]
    kc_ref = kc_b.cpu()
    for b in [0, 17, 63, int(torch.argmax(lens)), int(torch.argmin(lens))]:
        ref = oracle.attn_decode(q_r[b:b + 1], kc_ref[b:b + 1], vc_b[b:b + 1].cpu(), lens[b:b + 1])
        assert_close(o_b[b:b + 1], ref, torch.bfloat16, f"fused ragged step b={b} L={int(lens[b])}")


@pytest.mark.parametrize("style", [rgc.ROPE_HALF, rgc.ROPE_INTERLEAVED])
@pytest.mark.parametrize("D", [32, 64, 128])
@pytest.mark.parametrize("group", [1, 3, 8])
def test_fused_split_step_equals_prologue_then_decode_bit_for_bit(style, D, group):
    # 64 sequences of lengths up to 700 make more than 256 split workgroups,
    # so both forms take the split kernel (not the one-workgroup walk): with
    # group 8 two head subgroups share each new slot (only the first writes
    # it), with group 1 and 3 one workgroup covers the group.  The new slots
    # hold NaN canaries, so any read of a slot the step fills shows.
    Hkv = 2
    Hq = Hkv * group
    S_max = 700
    g = synth.generator(4000 + D + group + style)
    lens = synth.lengths(64, 1, S_max, g)
    lens[:6] = torch.tensor([1, 2, 128, 129, 256, 700], dtype=torch.int32)
    B = lens.numel()
    q, k_new, v_new, kc, vc = _inputs(B, Hq, Hkv, D, S_max, lens, seed=D * 10 + group + style + 77)
    dev = [t.cuda() for t in (q, k_new, v_new, kc, vc)]
    q_a, kn_a, vn_a, kc_a, vc_a = [t.clone() for t in dev]
    q_b, kn_b, vn_b, kc_b, vc_b = [t.clone() for t in dev]
    lens_g = lens.cuda()
    lse_a = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    lse_b = torch.empty_like(lse_a)
    o_a = _two_launch(q_a, kn_a, vn_a, kc_a, vc_a, lens_g, S_max, style, lse_a)
    o_b = rgc.gqa_attn_decode_rope_append(q_b, kn_b, vn_b, kc_b, vc_b, lens_g, S_max, style=style, lse=lse_b)
    assert torch.isfinite(o_b.float()).all(), "the fused step read a slot it was to fill"
    assert torch.equal(o_a.cpu().view(I16), o_b.cpu().view(I16))
    assert torch.equal(lse_a.cpu(), lse_b.cpu())
    assert torch.equal(kc_a.cpu().view(I16), kc_b.cpu().view(I16))
    assert torch.equal(vc_a.cpu().view(I16), vc_b.cpu().view(I16))
