"""Element-wise bound for the one-call layers that keep y_perm as block-scaled fp16.

Inside moe_forward (and its fp8 / MX forms) the W2 epilogue stores y_perm
block-scaled: for each row and 32-column block, s = floor(log2 max|v|) - 14
(clamped to [-127, 127], 0 for an all-zero block), and each value v becomes
fp16(v * 2^-s), nearest even. The step-wise path keeps the same fp32 values
(the same kernels accumulate them in the same order), so the two results y
differ only by that rounding and by the two fp32 combine sums:

* a value in fp16's normal range moves by at most 2^-11 |v|, one below it by
  at most 2^(s-25) (half the fp16 subnormal spacing, scaled back);
* each combine adds k weighted terms in slot order, every addition rounding
  by at most 2^-24 of the running sum, which stays within sum_j w_j |v_j|;
  the shared expert's term adds one more rounding of the result.

This holds for every element, where a bound in max|y_perm| only holds for
the largest ones: rounding toward zero instead of to nearest, or a scale
applied to the wrong block, breaks it on some element (tests/test_scaled16.py
plants both on the CPU). A scale taken over too many values does not: fp16
keeps 11 significant bits for any value within 2^28 of the block maximum, so
such a scale costs no precision; one taken over too few overflows to inf.
"""
import torch


def scaled16_bound(y_perm, A, inv, w, y_step):
    """Per-element bound on |y_one_call - y_step| (float64, shape of y_step).

    y_perm: the step-wise fp32 y_perm (its first A rows are the kept
    assignments, H % 32 == 0); inv, w: [T, k] routing maps of the same call;
    y_step: the step-wise layer output [T, H].
    """
    T, k = inv.shape
    H = y_perm.shape[1]
    assert H % 32 == 0
    yp = torch.cat([y_perm[:A].double(), torch.zeros((1, H), dtype=torch.float64, device=y_perm.device)])
    bm = yp.float().abs().view(-1, H // 32, 32).amax(-1)  # fp32 block maxima, as the kernel compares them
    _, ex = torch.frexp(bm)  # bm = m * 2^ex with m in [0.5, 1): floor(log2 bm) = ex - 1
    s = torch.where(bm > 0, (ex - 1 - 14).clamp(-127, 127), torch.zeros_like(ex)).double()
    err = 2.0 ** -11 * yp.abs() + torch.repeat_interleave(torch.exp2(s - 25), 32, dim=1)
    err[A] = 0.0
    rows = torch.where(inv >= 0, inv, torch.full_like(inv, A)).long()  # dropped slots read the zero row
    ww = w.double().unsqueeze(-1)
    round_terms = (ww * err[rows]).sum(1)
    mag = (ww * yp.abs()[rows]).sum(1)
    return round_terms + k * 2.0 ** -23 * mag + 2.0 ** -23 * y_step.double().abs()
