"""GPU parity: causal GQA prefill and cached decode against the fp64 oracle.

Inputs are seeded normal draws; every cache slot the call must not read holds
a NaN canary, so a read past a length shows up as a NaN in the result.
"""
import math

import pytest
import torch

import oracle
import rope_gqa_causal_amd as rgc
from rope_gqa_causal_amd import synth
from _util import assert_close

pytestmark = pytest.mark.gpu

LSE_TOL_BF16 = math.log1p(2.0 ** -9) + 1e-4


def _prefill_case(B, Sq, Hq, Hkv, D, dtype, q_start, S_max, seed):
    g = synth.generator(seed)
    q = synth.normal((B, Sq, Hq, D), g, dtype)
    kc, vc = synth.nan_cache(B, Hkv, S_max, D, dtype)
    for b in range(B):
        n = q_start[b] + Sq
        kc[b, :, :n] = synth.normal((Hkv, n, D), g, dtype)
        vc[b, :, :n] = synth.normal((Hkv, n, D), g, dtype)
    return q, kc, vc, torch.tensor(q_start, dtype=torch.int32)


PREFILL_CASES = [
    # B, Sq, Hq, Hkv, D, q_start,         S_max
    (2, 300, 6, 2, 128, [0, 0], 300),          # g=3, ragged tail of the 128-row tile
    (1, 256, 3, 3, 64, [0], 256),              # g=1 (MHA)
    (2, 200, 8, 1, 64, [0, 0], 224),           # g=8 (MQA), spare NaN slots
    (1, 160, 8, 2, 128, [0], 160),             # g=4 -> two heads per wave
    (1, 130, 6, 2, 32, [0], 130),              # D=32
    (2, 77, 12, 4, 64, [500, 31], 600),        # chunked prefill: rows start mid-cache
    (3, 1, 24, 8, 128, [0, 9, 1000], 1024),    # single-row blocks
    (1, 33, 2, 2, 128, [0], 40),
]


@pytest.mark.parametrize("case", PREFILL_CASES, ids=lambda c: f"B{c[0]}Sq{c[1]}H{c[2]}/{c[3]}D{c[4]}")
def test_prefill_bf16(case):
    B, Sq, Hq, Hkv, D, q_start, S_max = case
    q, kc, vc, qs = _prefill_case(B, Sq, Hq, Hkv, D, torch.bfloat16, q_start, S_max, sum(case[:5]))
    ref, ref_lse = oracle.attn(q, kc, vc, qs, want_lse=True)
    lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device="cuda")
    o = rgc.gqa_attn_prefill(q.cuda(), kc.cuda(), vc.cuda(), qs.cuda(), lse=lse)
    torch.cuda.synchronize()
    assert_close(o, ref, torch.bfloat16, "prefill bf16")
    # The bf16 kernels normalise by the sum of the bf16-rounded weights they
    # multiply V with; each weight carries a relative error <= 2^-9, so the
    # sum, and exp(lse), is off by at most that: |d lse| <= log(1 + 2^-9).
    assert (lse.cpu().double() - ref_lse).abs().max().item() < LSE_TOL_BF16


# Grids with more row blocks than compute units run persistent workgroups
# that walk several items each, prefetching the next item's Q and first
# tiles; sequences start at different cache slots, so neighbouring items
# differ in tile count.  Rows are checked by samples the oracle computes
# one block at a time.
PERSISTENT_CASES = [
    # B, Sq, Hq, Hkv, D, q_start,                 S_max
    (3, 1500, 24, 8, 128, [0, 300, 7], 1800),
    (6, 1000, 12, 4, 64, [0, 5, 100, 0, 63, 1], 1100),
    (8, 700, 16, 8, 32, [0, 1, 2, 3, 64, 65, 200, 0], 900),
]


@pytest.mark.parametrize("case", PERSISTENT_CASES, ids=lambda c: f"B{c[0]}Sq{c[1]}H{c[2]}/{c[3]}D{c[4]}")
def test_prefill_persistent_grid_sampled_rows(case):
    B, Sq, Hq, Hkv, D, q_start, S_max = case
    q, kc, vc, qs = _prefill_case(B, Sq, Hq, Hkv, D, torch.bfloat16, q_start, S_max, Sq + D)
    lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device="cuda")
    o = rgc.gqa_attn_prefill(q.cuda(), kc.cuda(), vc.cuda(), qs.cuda(), lse=lse).cpu()
    lse = lse.cpu().double()
    sg = synth.generator(Sq)
    for b in range(B):
        s0 = int(torch.randint(0, Sq - 16, (1,), generator=sg))
        for lo in (0, s0, Sq - 16):
            rows = slice(lo, lo + 16)
            ref, ref_lse = oracle.attn(q[b:b + 1, rows], kc[b:b + 1], vc[b:b + 1],
                                       torch.tensor([q_start[b] + lo], dtype=torch.int32), want_lse=True)
            assert_close(o[b:b + 1, rows], ref, torch.bfloat16, f"persistent prefill b={b} rows {lo}")
            assert (lse[b:b + 1, :, rows] - ref_lse).abs().max().item() < LSE_TOL_BF16


@pytest.mark.parametrize("case", [(1, 16, 4, 2, 32, [0], 24), (2, 70, 6, 3, 64, [0, 5], 80),
                                  (1, 40, 8, 2, 128, [3], 48)])
def test_prefill_fp32(case):
    B, Sq, Hq, Hkv, D, q_start, S_max = case
    q, kc, vc, qs = _prefill_case(B, Sq, Hq, Hkv, D, torch.float32, q_start, S_max, 11)
    ref, ref_lse = oracle.attn(q, kc, vc, qs, want_lse=True)
    lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device="cuda")
    o = rgc.gqa_attn_prefill(q.cuda(), kc.cuda(), vc.cuda(), qs.cuda(), lse=lse)
    assert_close(o, ref, torch.float32, "prefill fp32")
    assert (lse.cpu().double() - ref_lse).abs().max().item() < 1e-5


def test_prefill_on_bshd_tensors_standing_in_for_a_cache():
    # k, v in [B,S,Hkv,D] layout passed through strides (no cache copy).
    B, S, Hq, Hkv, D = 2, 150, 6, 2, 128
    g = synth.generator(5)
    q, k, v = synth.qkv(B, S, Hq, Hkv, D, g)
    ref = oracle.attn(q, k.transpose(1, 2), v.transpose(1, 2))
    o = rgc.gqa_attn_prefill(q.cuda(), k.cuda().transpose(1, 2), v.cuda().transpose(1, 2))
    assert_close(o, ref, torch.bfloat16, "bshd prefill")


def _decode_case(B, Hq, Hkv, D, lens, S_max, dtype, seed):
    g = synth.generator(seed)
    kc, vc = synth.nan_cache(B, Hkv, S_max, D, dtype)
    for b, L in enumerate(lens):
        kc[b, :, :L] = synth.normal((Hkv, L, D), g, dtype)
        vc[b, :, :L] = synth.normal((Hkv, L, D), g, dtype)
    q = synth.normal((B, Hq, D), g, dtype)
    return q, kc, vc, torch.tensor(lens, dtype=torch.int32)


DECODE_CASES = [
    # Hq, Hkv, D, lens, S_max
    (24, 8, 128, [1, 255, 256, 257, 600, 2049, 1024, 3], 2080),
    (12, 4, 64, [513, 612, 1, 700], 720),
    (4, 2, 32, [17, 24, 300], 320),
    (16, 2, 128, [900, 64], 1000),            # g=8 -> two head subgroups
    (5, 5, 64, [100, 1500], 1600),            # g=1
    # Batches with at least 1024 workgroups of 256-key chunks take the
    # longer-chunk kernels (64 keys per wave).
    (8, 8, 128, [2048, 1, 255, 256, 257, 1000, 1777, 513, 64, 2047, 1500, 300, 129, 2000, 900, 1200], 2048),
    (16, 8, 64, [2048, 17, 256, 257, 511, 512, 1999, 1024, 700, 1, 80, 1300, 1800, 640, 333, 2040], 2060),
]


@pytest.mark.parametrize("case", DECODE_CASES, ids=lambda c: f"H{c[0]}/{c[1]}D{c[2]}")
def test_decode_bf16(case):
    Hq, Hkv, D, lens, S_max = case
    q, kc, vc, L = _decode_case(len(lens), Hq, Hkv, D, lens, S_max, torch.bfloat16, Hq + D)
    ref, ref_lse = oracle.attn_decode(q, kc, vc, L, want_lse=True)
    lse = torch.empty((len(lens), Hq), dtype=torch.float32, device="cuda")
    o = rgc.gqa_attn_decode(q.cuda(), kc.cuda(), vc.cuda(), L.cuda(), max(lens), lse=lse)
    assert_close(o, ref, torch.bfloat16, "decode bf16")
    assert (lse.cpu().double() - ref_lse).abs().max().item() < 1e-3


@pytest.mark.parametrize("D,longest", [(32, 3072), (64, 1536), (128, 768)])
def test_decode_walk_at_its_longest_and_split_one_key_past_it(D, longest):
    # A small grid walks each sequence in one workgroup of 12 waves for up to
    # two passes (12 x 128, 12 x 64 or 12 x 32 keys per pass at head dim 32,
    # 64, 128); one key more takes the split-K kernel and its merge.  Both
    # against the oracle, and against each other.
    Hq, Hkv = 8, 2
    lens = [longest, longest // 2 + 1, 256, 1]
    q, kc, vc, L = _decode_case(len(lens), Hq, Hkv, D, lens, longest + 1, torch.bfloat16, 77 + D)
    ref = oracle.attn_decode(q, kc, vc, L)
    qg, kg, vg, Lg = q.cuda(), kc.cuda(), vc.cuda(), L.cuda()
    walk = rgc.gqa_attn_decode(qg, kg, vg, Lg, longest)
    split = rgc.gqa_attn_decode(qg, kg, vg, Lg, longest + 1)
    assert_close(walk, ref, torch.bfloat16, "decode walk, 8 chunks")
    assert_close(split, ref, torch.bfloat16, "decode split, 2049 keys")
    assert (walk.float() - split.float()).abs().max().item() <= 2.0 ** -6


def test_decode_fp32():
    q, kc, vc, L = _decode_case(3, 4, 2, 32, [1, 17, 24], 24, torch.float32, 3)
    ref = oracle.attn_decode(q, kc, vc, L)
    o = rgc.gqa_attn_decode(q.cuda(), kc.cuda(), vc.cuda(), L.cuda(), 24)
    assert_close(o, ref, torch.float32, "decode fp32")


def _rising(x, u, step):
    """Adds step * j * u to row j of x [..., S, D]: scores against queries
    that point along u grow with the key's position."""
    S = x.shape[-2]
    ramp = torch.arange(S, dtype=torch.float64)[:, None] * step * u.double()[None, :]
    return (x.double() + ramp).to(x.dtype)


@pytest.mark.parametrize("dtype,D,growth", [(torch.bfloat16, 128, 8.0), (torch.bfloat16, 64, 8.0),
                                            (torch.float32, 64, 2.0)])
def test_prefill_and_decode_when_the_running_max_rises_tile_after_tile(dtype, D, growth):
    # Keys grow along the sequence in the queries' direction by `growth` (in
    # units of the scaled score) every 64 keys, so almost every later tile
    # holds a new row maximum -- for the bf16 kernels, past their rescale
    # threshold of 2^8 (5.5 score units): the rare raise-and-rescale path
    # runs on most tiles of most rows, in prefill and in both decode forms
    # (the one-workgroup walk, which rescales across its chunks, at batch 1;
    # the split-K kernel and its merge with the batch repeated 64 times).  The fp32 case grows more slowly: scores rounded in
    # fp32 carry an error of |s| 2^-24, which logits of ~65 would lift past
    # the 1e-5 bar through the exponentials; at ~16 they stay well inside.
    B, S, Hq, Hkv = 1, 520, 4, 2
    g = synth.generator(41 + D)
    u = synth.normal((D,), g, torch.float64)
    u = u / u.norm()
    q = (synth.normal((B, S, Hq, D), g, torch.float64) * 0.3 + 2.0 * u).to(dtype)
    step = growth / (64 * 2.0 / math.sqrt(D))
    kc = torch.empty((B, Hkv, S, D), dtype=dtype)
    vc = synth.normal((B, Hkv, S, D), g, dtype)
    for h in range(Hkv):
        kc[0, h] = _rising(synth.normal((S, D), g, dtype), u, step)
    qs = torch.zeros(B, dtype=torch.int32)
    ref, ref_lse = oracle.attn(q, kc, vc, qs, want_lse=True)
    lse = torch.empty((B, Hq, S), dtype=torch.float32, device="cuda")
    o = rgc.gqa_attn_prefill(q.cuda(), kc.cuda(), vc.cuda(), qs.cuda(), lse=lse)
    assert_close(o, ref, dtype, "prefill, rising scores")
    lse_tol = LSE_TOL_BF16 if dtype == torch.bfloat16 else 1e-5
    assert (lse.cpu().double() - ref_lse).abs().max().item() < lse_tol
    # Decode of the last row over the whole cache.
    lens = torch.tensor([S], dtype=torch.int32)
    q1 = q[:, -1].contiguous()
    ref1 = oracle.attn_decode(q1, kc, vc, lens)
    o1 = rgc.gqa_attn_decode(q1.cuda(), kc.cuda(), vc.cuda(), lens.cuda(), S)
    assert_close(o1, ref1, dtype, "decode, rising scores")
    if dtype == torch.bfloat16:
        R = 64
        o64 = rgc.gqa_attn_decode(q1.repeat(R, 1, 1).cuda(), kc.repeat(R, 1, 1, 1).cuda(), vc.repeat(R, 1, 1, 1).cuda(),
                                  lens.repeat(R).cuda(), S)
        assert_close(o64, ref1.repeat(R, 1, 1), dtype, "split-K decode, rising scores")


def test_decode_equals_prefill_last_row_and_gqa_equals_mha_on_gpu():
    # Two GPU-side invariants: the decode row equals the prefill row at the
    # same slot; GQA equals MHA over repeated KV heads.
    B, Hq, Hkv, D, S = 2, 6, 2, 128, 333
    g = synth.generator(21)
    q, k, v = synth.qkv(B, S, Hq, Hkv, D, g)
    kc, vc = k.transpose(1, 2).contiguous().cuda(), v.transpose(1, 2).contiguous().cuda()
    o_pre = rgc.gqa_attn_prefill(q.cuda(), kc, vc)
    lens = torch.full((B,), S, dtype=torch.int32, device="cuda")
    o_dec = rgc.gqa_attn_decode(q[:, -1].contiguous().cuda(), kc, vc, lens, S)
    assert_close(o_dec, o_pre[:, -1].double().cpu(), torch.bfloat16, "decode vs prefill")
    kr = kc.repeat_interleave(Hq // Hkv, dim=1)
    vr = vc.repeat_interleave(Hq // Hkv, dim=1)
    o_mha = rgc.gqa_attn_prefill(q.cuda(), kr, vr)
    assert_close(o_mha, o_pre.double().cpu(), torch.bfloat16, "gqa vs mha")


def test_future_rows_cannot_change_earlier_outputs_bitwise():
    B, S, Hq, Hkv, D = 1, 256, 6, 2, 128
    g = synth.generator(31)
    q, k, v = synth.qkv(B, S, Hq, Hkv, D, g)
    kc, vc = k.transpose(1, 2).contiguous(), v.transpose(1, 2).contiguous()
    o1 = rgc.gqa_attn_prefill(q.cuda(), kc.cuda(), vc.cuda()).cpu()
    kc2, vc2 = kc.clone(), vc.clone()
    kc2[:, :, 200:] = synth.normal((B, Hkv, S - 200, D), g) * 4
    vc2[:, :, 200:] = synth.normal((B, Hkv, S - 200, D), g) * 4
    o2 = rgc.gqa_attn_prefill(q.cuda(), kc2.cuda(), vc2.cuda()).cpu()
    assert torch.equal(o1[:, :200].view(torch.int16), o2[:, :200].view(torch.int16))
    o3 = rgc.gqa_attn_prefill(q.cuda(), kc.cuda(), vc.cuda()).cpu()
    assert torch.equal(o1.view(torch.int16), o3.view(torch.int16))  # run-to-run determinism


def test_device_side_capacity_violations_give_nan_rows_and_a_flag():
    B, Hq, Hkv, D, S_max = 2, 4, 2, 64, 64
    q, kc, vc, L = _decode_case(B, Hq, Hkv, D, [10, 64], S_max, torch.bfloat16, 41)
    bad = torch.tensor([10, 65], dtype=torch.int32, device="cuda")     # 65 > S_max
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    o = rgc.gqa_attn_decode(q.cuda(), kc.cuda(), vc.cuda(), bad, S_max, err_flag=err)
    assert err.item() == 1
    assert torch.isnan(o[1].float()).all() and torch.isfinite(o[0].float()).all()
    qp = synth.normal((B, 8, Hq, D), synth.generator(42))
    err.zero_()
    o = rgc.gqa_attn_prefill(qp.cuda(), kc.cuda(), vc.cuda(),
                             torch.tensor([0, 60], dtype=torch.int32, device="cuda"), err_flag=err)
    assert err.item() == 1
    assert torch.isnan(o[1].float()).all() and torch.isfinite(o[0].float()).all()
