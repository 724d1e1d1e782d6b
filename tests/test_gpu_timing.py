"""GPU: the instrumented build's per-kernel timing records each kernel of a
call apart, and only while switched on.  Also shows which decode form a shape takes: a
small grid walks each sequence in one workgroup (one kernel), a large one
splits the cache (split kernel, then the merge)."""
import pytest
import torch

import rope_gqa_causal_amd as rgc
from rope_gqa_causal_amd import synth

pytestmark = pytest.mark.gpu


def _decode_setup(B, Hq, Hkv, D, S_max, seed):
    g = synth.generator(seed)
    kc, vc = synth.filled_cache(B, Hkv, S_max, D, g)
    q = synth.normal((B, Hq, D), g).cuda()
    lens = synth.lengths(B, 1, S_max, g).cuda()
    return q, kc.cuda(), vc.cuda(), lens, rgc.decode_workspace(B, Hq, Hkv, D, S_max)


@pytest.mark.parametrize("B,Hq,Hkv,S_max,kernels", [
    (4, 6, 2, 760, {"decode_loop_kernel"}),                                 # 4 x 2 units, two passes
    (40, 24, 8, 1200, {"decode_split_kernel", "decode_combine_kernel"}),   # 320 units: split-K
])
def test_decode_kernels_are_timed_apart_and_only_while_on(B, Hq, Hkv, S_max, kernels):
    q, kc, vc, lens, ws = _decode_setup(B, Hq, Hkv, 128, S_max, 21)
    rgc.timing_report()  # clear
    ref = rgc.gqa_attn_decode(q, kc, vc, lens, S_max, ws)  # product build: not recorded
    with rgc.kernel_timing():
        for _ in range(3):
            o = rgc.gqa_attn_decode(q, kc, vc, lens, S_max, ws)
    rgc.gqa_attn_decode(q, kc, vc, lens, S_max, ws)  # off again
    torch.cuda.synchronize()
    assert torch.equal(o, ref)  # the instrumented build runs the same kernels
    rep = rgc.timing_report()
    assert set(rep) == kernels, rep
    for name, (calls, us) in rep.items():
        assert calls == 3, (name, calls)
        assert 0.0 < us < 3e5, (name, us)
    assert rgc.timing_report() == {}  # the report cleared the record
