"""GPU parity: cached decode of differential attention against the fp64
oracle (the oracle's differential attention with one query row per sequence
at slot L - 1, page "750美元从零训练3个LLM：一位开发者的实战复盘", section
V2).  Cache slots at and past each sequence's length hold NaN canaries, so a
read past a length poisons the output."""
import pytest
import torch

import oracle
import rope_gqa_causal_amd as rgc
from rope_gqa_causal_amd import synth
from _util import assert_close

pytestmark = pytest.mark.gpu


def _case(B, Hq, Hkv, D, lens, S_max, seed):
    g = synth.generator(seed)
    q1 = synth.normal((B, Hq, D), g)
    q2 = synth.normal((B, Hq, D), g)
    caches = []
    for _ in range(3):  # k1, k2, v
        c = torch.full((B, Hkv, S_max, D), float("nan"), dtype=torch.bfloat16)
        for b in range(B):
            c[b, :, :lens[b]] = synth.normal((Hkv, lens[b], D), g)
        caches.append(c)
    return q1, q2, caches, torch.tensor(lens, dtype=torch.int32)


def _oracle(q1, q2, caches, lens, lam):
    # one query row per sequence at slot L - 1 over keys 0..L-1
    return oracle.diff_attn(q1[:, None], q2[:, None], caches[0], caches[1], caches[2], lam, lens - 1)[:, 0]


CASES = [
    # B, Hq, Hkv, D, lens, S_max, lambda
    (3, 4, 2, 64, [1, 128, 129], 130, 0.8),             # one key, one chunk, chunk + 1
    (4, 16, 8, 64, [1000, 257, 640, 1024], 1024, 0.8),  # the differential workload's heads
    (2, 6, 2, 64, [300, 77], 300, 0.5),                 # group 3: one head per workgroup
    (2, 8, 2, 128, [700, 129], 700, 0.8),               # group 4, head dim 128
    (2, 4, 4, 32, [513, 256], 600, 1.25),               # group 1, head dim 32, lambda above one
    (5, 2, 1, 64, [2, 31, 33, 500, 1999], 2000, 0.8),   # many chunks
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"B{c[0]}H{c[1]}/{c[2]}D{c[3]}l{c[6]}")
def test_diff_decode_matches_oracle(case):
    B, Hq, Hkv, D, lens, S_max, lam = case
    q1, q2, caches, L = _case(B, Hq, Hkv, D, lens, S_max, B + Hq + D)
    ref = _oracle(q1, q2, caches, L, lam)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    o = rgc.diff_attn_decode(q1.cuda(), q2.cuda(), *(c.cuda() for c in caches), L.cuda(), lam, S_max,
                             err_flag=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    assert_close(o, ref, torch.bfloat16, "differential decode")


def test_lambda_zero_is_the_plain_decode_of_the_first_map():
    B, Hq, Hkv, D, S_max = 4, 16, 8, 64, 900
    lens = [900, 1, 400, 257]
    q1, q2, caches, L = _case(B, Hq, Hkv, D, lens, S_max, 11)
    g = [t.cuda() for t in (q1, q2, *caches)]
    zero = rgc.diff_attn_decode(g[0], g[1], g[2], g[3], g[4], L.cuda(), 0.0, S_max).cpu()
    plain = rgc.gqa_attn_decode(g[0], g[2], g[4], L.cuda(), S_max).cpu()
    ref = oracle.attn_decode(q1, caches[0], caches[2], L)
    assert_close(zero, ref, torch.bfloat16, "lambda 0 against the plain oracle decode")
    assert_close(plain, ref, torch.bfloat16, "plain decode")


def test_invalid_lengths_give_nan_rows_and_the_flag():
    B, Hq, Hkv, D, S_max = 3, 4, 2, 64, 200
    q1, q2, caches, L = _case(B, Hq, Hkv, D, [50, 150, 200], S_max, 12)
    bad = torch.tensor([50, 0, 150], dtype=torch.int32)  # a zero length
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    o = rgc.diff_attn_decode(q1.cuda(), q2.cuda(), *(c.cuda() for c in caches), bad.cuda(), 0.8, 150,
                             err_flag=err).cpu()
    torch.cuda.synchronize()
    assert int(err.item()) == 1
    assert torch.isnan(o[1].float()).all()
    ref = _oracle(q1[[0, 2]], q2[[0, 2]], [c[[0, 2]] for c in caches], bad[[0, 2]], 0.8)
    assert_close(o[[0, 2]], ref, torch.bfloat16, "valid rows beside an invalid one")


@pytest.mark.parametrize("seed", [5, 105, 205])
def test_ragged_batch_of_the_bench_sampled(seed):
    # 64 sequences of lengths U{256..2048}, 16 q / 8 KV heads, D 64: the
    # launch the bench times; eight sequences are checked against the oracle
    B, Hq, Hkv, D = 64, 16, 8, 64
    g = synth.generator(seed)
    lens = synth.lengths(B, 256, 2048, g)
    S_max = 2048
    q1 = synth.normal((B, Hq, D), g)
    q2 = synth.normal((B, Hq, D), g)
    caches = [synth.normal((B, Hkv, S_max, D), g) for _ in range(3)]
    o = rgc.diff_attn_decode(q1.cuda(), q2.cuda(), *(c.cuda() for c in caches), lens.cuda(), 0.8, S_max).cpu()
    pick = torch.randperm(B, generator=g)[:8]
    ref = _oracle(q1[pick], q2[pick], [c[pick] for c in caches], lens[pick], 0.8)
    assert_close(o[pick], ref, torch.bfloat16, "sampled sequences of the ragged differential decode")
