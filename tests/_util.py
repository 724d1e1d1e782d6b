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
# Gradients (attention backward) sum many heads' and rows' contributions and
# reach magnitudes where rounding the result to bf16 alone costs up to half
# an ulp, 2^-8 |x|: their per-element bound adds that to the bf16 bar.
BF16_ROUND_REL = 2.0 ** -8


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


def assert_close_grad(got, ref, what=""):
    """bf16 gradient parity: |got - ref| <= 2e-2 + 2^-8 |ref| per element and
    ||got - ref|| <= 5e-3 max(||ref||, 2e-2 sqrt(n))."""
    g = got.detach().to("cpu", torch.float64)
    r = ref.detach().to("cpu", torch.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    assert torch.isfinite(g).all(), "non-finite values in the GPU result"
    d = (g - r).abs()
    excess = (d - BF16_ROUND_REL * r.abs()).max().item() if d.numel() else 0.0
    # A reference that vanishes (a one-token sequence has dK = 0 exactly) is
    # measured against the absolute bar's scale instead of its own norm.
    rel = (g - r).norm().item() / max(r.norm().item(), BF16_MAX_ABS * d.numel() ** 0.5)
    assert excess <= BF16_MAX_ABS and rel <= BF16_REL_L2, \
        f"{what}: bf16 gradient excess {excess:.3e} (max-abs {d.max().item():.3e}), rel-L2 {rel:.3e}"
    return excess, rel


def gpu_available():
    return torch.cuda.is_available()
