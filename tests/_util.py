"""Comparison helpers and tolerances for GPU-vs-oracle parity tests.

Tolerances (stated once, used everywhere):
  * fp32 paths: max |gpu - oracle| <= 1e-5;
  * bf16 paths: max |gpu - oracle| <= 2e-2 and ||gpu - oracle|| / ||oracle|| <= 5e-3;
  * cache indexing: bit-exact.
The oracle runs in fp64 on exactly the inputs the GPU saw.
"""
import torch

FP32_MAX_ABS = 1e-5
BF16_MAX_ABS = 2e-2
BF16_REL_L2 = 5e-3


def errors(got, ref):
    g = got.detach().to("cpu", torch.float64)
    r = ref.detach().to("cpu", torch.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    assert torch.isfinite(g).all(), "non-finite values in the GPU result"
    d = g - r
    max_abs = d.abs().max().item() if d.numel() else 0.0
    denom = r.norm().item()
    rel = d.norm().item() / denom if denom > 0 else d.norm().item()
    return max_abs, rel


def assert_close(got, ref, dtype, what=""):
    max_abs, rel = errors(got, ref)
    if dtype == torch.float32:
        assert max_abs <= FP32_MAX_ABS, f"{what}: fp32 max-abs {max_abs:.3e}"
    else:
        assert max_abs <= BF16_MAX_ABS and rel <= BF16_REL_L2, \
            f"{what}: bf16 max-abs {max_abs:.3e}, rel-L2 {rel:.3e}"
    return max_abs, rel


def gpu_available():
    return torch.cuda.is_available()
