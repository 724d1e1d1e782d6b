"""GPU: the library's per-kernel timing records each kernel of a call apart
(the decode's split kernel and its merge), and only while switched on."""
import pytest
import torch

import rope_gqa_causal_amd as rgc
from rope_gqa_causal_amd import synth

pytestmark = pytest.mark.gpu


def test_decode_kernels_are_timed_apart_and_only_while_on():
    B, Hq, Hkv, D, S_max = 4, 6, 2, 128, 1200
    g = synth.generator(21)
    kc, vc = synth.filled_cache(B, Hkv, S_max, D, g)
    q = synth.normal((B, Hq, D), g).cuda()
    kc, vc = kc.cuda(), vc.cuda()
    lens = torch.tensor([1200, 700, 64, 1], dtype=torch.int32).cuda()
    ws = rgc.decode_workspace(B, Hq, Hkv, D, S_max)
    rgc.timing_report()  # clear
    rgc.gqa_attn_decode(q, kc, vc, lens, S_max, ws)  # timing off: not recorded
    rgc.timing_enable(True)
    try:
        for _ in range(3):
            rgc.gqa_attn_decode(q, kc, vc, lens, S_max, ws)
    finally:
        rgc.timing_enable(False)
    rgc.gqa_attn_decode(q, kc, vc, lens, S_max, ws)  # off again
    rep = rgc.timing_report()
    assert set(rep) == {"decode_split_kernel", "decode_combine_kernel"}, rep
    for name, (calls, us) in rep.items():
        assert calls == 3, (name, calls)
        assert 0.0 < us < 3e5, (name, us)
    assert rgc.timing_report() == {}  # the report cleared the record
