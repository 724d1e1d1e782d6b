"""GPU parity: causal differential attention against the fp64 oracle.

o = (softmax(s q1 K1^T) - lambda softmax(s q2 K2^T)) V.  Inputs are seeded
normal draws; cache slots past each workgroup's last key hold NaN canaries.
"""
import pytest
import torch

import oracle
import rope_gqa_causal_amd as rgc
from rope_gqa_causal_amd import synth
from _util import assert_close

pytestmark = pytest.mark.gpu

D = 64


def _diff_case(B, Sq, Hq, Hkv, q_start, S_max, seed, D=D):
    g = synth.generator(seed)
    q1 = synth.normal((B, Sq, Hq, D), g)
    q2 = synth.normal((B, Sq, Hq, D), g)
    caches = []
    for _ in range(3):  # k1, k2, v
        c = torch.full((B, Hkv, S_max, D), float("nan"), dtype=torch.bfloat16)
        for b in range(B):
            n = q_start[b] + Sq
            c[b, :, :n] = synth.normal((Hkv, n, D), g)
        caches.append(c)
    return q1, q2, caches[0], caches[1], caches[2], torch.tensor(q_start, dtype=torch.int32)


DIFF_CASES = [
    # B, Sq, Hq, Hkv, q_start, S_max, lambda
    (2, 300, 4, 2, [0, 0], 300, 0.8),        # g=2, ragged tail of a 128-position tile
    (1, 257, 8, 8, [0], 260, 0.8),           # g=1, one row past a tile
    (2, 130, 6, 1, [0, 0], 140, 0.5),        # g=6 (one KV head)
    (2, 77, 16, 8, [500, 31], 600, 0.8),     # rows start mid-cache
    (3, 1, 4, 2, [0, 9, 100], 128, 0.8),     # single rows
    (1, 65, 2, 1, [0], 65, 1.25),            # lambda above one
]


@pytest.mark.parametrize("case", DIFF_CASES, ids=lambda c: f"B{c[0]}Sq{c[1]}H{c[2]}/{c[3]}l{c[6]}")
def test_diff_attn_bf16(case):
    B, Sq, Hq, Hkv, q_start, S_max, lam = case
    q1, q2, k1, k2, v, qs = _diff_case(B, Sq, Hq, Hkv, q_start, S_max, Sq + Hq)
    ref = oracle.diff_attn(q1, q2, k1, k2, v, lam, qs)
    o = rgc.diff_attn_prefill(q1.cuda(), q2.cuda(), k1.cuda(), k2.cuda(), v.cuda(), lam, qs.cuda())
    torch.cuda.synchronize()
    assert_close(o, ref, torch.bfloat16, "diff attention")


def test_lambda_zero_is_plain_attention_and_equal_maps_scale_by_one_minus_lambda():
    B, Sq, Hq, Hkv = 2, 200, 4, 2
    q1, q2, k1, k2, v, qs = _diff_case(B, Sq, Hq, Hkv, [0, 0], Sq, 7)
    g = [t.cuda() for t in (q1, q2, k1, k2, v)]
    plain = oracle.attn(q1, k1, v, qs)
    # lambda = 0: the first map alone, i.e. plain causal attention.
    zero = rgc.diff_attn_prefill(g[0], g[1], g[2], g[3], g[4], 0.0).cpu()
    assert_close(zero, plain, torch.bfloat16, "lambda 0")
    # Two equal maps: (1 - lambda) times plain attention.
    same = rgc.diff_attn_prefill(g[0], g[0], g[2], g[2], g[4], 0.8).cpu()
    assert_close(same, plain.double() * 0.2, torch.bfloat16, "equal maps")


@pytest.mark.parametrize("seed_off", [0, 100, 200])
def test_diff_workload_full_size_sampled_rows(seed_off):
    # The differential workload (B 4 x 1024 tokens, 16 q / 8 KV heads, D 64,
    # lambda 0.8) launched as the bench times it; the oracle recomputes
    # sampled row blocks (rows start mid-sequence through q_start): the
    # first rows, a block across the 128-position tile boundary at 512, and
    # the last rows, whose workgroups are the heaviest.
    w = synth.WORKLOADS["diff"]
    g = synth.generator(w.seed + seed_off)
    q1 = synth.normal((w.B, w.S, w.Hq, w.D), g)
    q2 = synth.normal((w.B, w.S, w.Hq, w.D), g)
    k1 = synth.normal((w.B, w.Hkv, w.S, w.D), g)
    k2 = synth.normal((w.B, w.Hkv, w.S, w.D), g)
    v = synth.normal((w.B, w.Hkv, w.S, w.D), g)
    o = rgc.diff_attn_prefill(q1.cuda(), q2.cuda(), k1.cuda(), k2.cuda(), v.cuda(), w.lam).cpu()
    for s0, s1 in ((0, 40), (500, 530), (990, 1024)) if seed_off == 0 else ((100, 140), (630, 660), (1000, 1024)):
        qs = torch.full((w.B,), s0, dtype=torch.int32)
        ref = oracle.diff_attn(q1[:, s0:s1].contiguous(), q2[:, s0:s1].contiguous(), k1, k2, v, w.lam, qs)
        assert_close(o[:, s0:s1], ref, torch.bfloat16, f"diff rows {s0}..{s1}")


def test_diff_capacity_violation_gives_nan_rows_and_a_flag():
    q1, q2, k1, k2, v, _ = _diff_case(2, 8, 4, 2, [0, 0], 64, 3)
    for c in (k1, k2, v):
        c[:, :, 8:] = 0.0
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    bad = torch.tensor([0, 60], dtype=torch.int32, device="cuda")  # 60 + 8 > 64
    o = rgc.diff_attn_prefill(q1.cuda(), q2.cuda(), k1.cuda(), k2.cuda(), v.cuda(), 0.8, bad, err_flag=err)
    assert err.item() == 1
    assert torch.isnan(o[1].float()).all() and torch.isfinite(o[0].float()).all()


# Head dims other than 64 run as two launches of the causal prefill kernel,
# the second adding -lambda times its output into o.
TWO_PASS_CASES = [
    # D, B, Sq, Hq, Hkv, q_start, S_max, lambda
    (128, 2, 300, 6, 2, [0, 0], 300, 0.8),    # g=3, ragged tail
    (128, 2, 77, 4, 4, [500, 31], 600, 0.8),  # rows start mid-cache
    (32, 1, 257, 8, 2, [0], 260, 1.25),       # g=4, lambda above one
    (32, 3, 1, 4, 2, [0, 9, 100], 128, 0.5),  # single rows
]


@pytest.mark.parametrize("case", TWO_PASS_CASES, ids=lambda c: f"D{c[0]}B{c[1]}Sq{c[2]}H{c[3]}/{c[4]}")
def test_diff_attn_two_pass_head_dims(case):
    Dh, B, Sq, Hq, Hkv, q_start, S_max, lam = case
    q1, q2, k1, k2, v, qs = _diff_case(B, Sq, Hq, Hkv, q_start, S_max, Sq + Hq + Dh, D=Dh)
    print(f"[diff two-pass] D={Dh} B={B} Sq={Sq} H={Hq}/{Hkv}", flush=True)
    ref = oracle.diff_attn(q1, q2, k1, k2, v, lam, qs)
    g = [t.cuda() for t in (q1, q2, k1, k2, v)]
    o = rgc.diff_attn_prefill(g[0], g[1], g[2], g[3], g[4], lam, qs.cuda())
    torch.cuda.synchronize()
    assert_close(o, ref, torch.bfloat16, f"diff attention, D {Dh}")
    # lambda = 0 leaves the first pass's output untouched: bit for bit the
    # causal prefill of (q1, K1, V).
    zero = rgc.diff_attn_prefill(g[0], g[1], g[2], g[3], g[4], 0.0, qs.cuda())
    plain = rgc.gqa_attn_prefill(g[0], g[2], g[4], qs.cuda())
    torch.cuda.synchronize()
    assert torch.equal(zero.view(torch.int16), plain.view(torch.int16))
