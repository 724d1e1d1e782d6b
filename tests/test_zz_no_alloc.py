"""GPU: the allocation-free one-launch decode step, whose chunk partials go
to the library's own per-GPU array, gives the output, lse and caches of the
workspace entry point bit for bit, on calls in a row whose inputs shrink
(the array keeps the previous call's partials; every slot a call reads is
written by that call first)."""
import pytest
import torch

import rope_gqa_causal_amd as rgc
from rope_gqa_causal_amd import synth

pytestmark = pytest.mark.gpu

# (B, Hq, Hkv, D, S_max, seed): the ragged-decode shape (split-K, 26,112
# partial slots), a smaller split-K shape, and a batch-1 shape that walks
# each sequence in one workgroup (no partials at all).
CASES = [(64, 24, 8, 128, 2080, 31), (12, 12, 4, 64, 700, 32), (1, 12, 4, 64, 612, 33)]


def _inputs(B, Hq, Hkv, D, S_max, seed):
    g = synth.generator(seed)
    kc, vc = synth.filled_cache(B, Hkv, S_max, D, g)
    q = synth.normal((B, Hq, D), g)
    kn = synth.normal((B, Hkv, D), g)
    vn = synth.normal((B, Hkv, D), g)
    lens = synth.lengths(B, 1, S_max, g)
    return [t.cuda() for t in (q, kn, vn, kc, vc, lens)]


def test_static_scratch_step_equals_the_workspace_step_on_shrinking_calls():
    for B, Hq, Hkv, D, S_max, seed in CASES:
        print(f"[no-alloc] B={B} Hq={Hq} Hkv={Hkv} D={D} S_max={S_max} seed={seed}", flush=True)
        q, kn, vn, kc, vc, lens = _inputs(B, Hq, Hkv, D, S_max, seed)
        kc_a, vc_a, kc_b, vc_b = kc.clone(), vc.clone(), kc.clone(), vc.clone()
        lse_a = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
        lse_b = torch.empty_like(lse_a)
        err = torch.zeros(1, dtype=torch.int32, device="cuda")
        ws = rgc.decode_workspace(B, Hq, Hkv, D, S_max)
        o_a = rgc.gqa_attn_decode_rope_append(q, kn, vn, kc_a, vc_a, lens, S_max, ws, lse=lse_a, err_flag=err)
        o_b = rgc.gqa_attn_decode_rope_append_static(q, kn, vn, kc_b, vc_b, lens, S_max, lse=lse_b, err_flag=err)
        torch.cuda.synchronize()
        assert int(err.item()) == 0
        assert torch.isfinite(o_b.float()).all()
        assert torch.equal(o_a, o_b)
        assert torch.equal(lse_a, lse_b)
        assert torch.equal(kc_a, kc_b) and torch.equal(vc_a, vc_b)
