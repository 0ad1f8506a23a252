"""The element-wise bound of tests/scaled16.py, checked on a CPU simulation of
the block-scaled fp16 rounding: the rounding as specified stays within it, and
two planted mistakes (rounding toward zero; each block decoded with its left
neighbour's scale) break it. The first of them stays within the coarser bound
2^-10 * max|y_perm|.
"""
import torch

from tests.scaled16 import scaled16_bound

T, K, H = 50, 3, 96


def _case(seed=0):
    g = torch.Generator().manual_seed(seed)
    # blocks of very different magnitudes, so scales differ from block to block
    yp = torch.randn(T * K, H, generator=g) * torch.exp(
        2 * torch.randn(T * K, H // 32, generator=g)).repeat_interleave(32, 1)
    A = T * K - 7
    inv = torch.randperm(T * K, generator=g).view(T, K).int()
    inv[inv >= A] = -1
    w = torch.rand(T, K, generator=g)
    w = w / w.sum(1, keepdim=True)
    w[inv < 0] = 0
    return yp, A, inv, w


def _combine(Y, inv, w):
    out = torch.zeros(T, H)
    for j in range(K):
        r = inv[:, j].long()
        out = out + w[:, j:j + 1] * torch.where((r >= 0)[:, None], Y[r.clamp(min=0)], torch.zeros(1, H))
    return out


def _exponents(Y):
    bm = Y.abs().view(-1, H // 32, 32).amax(-1)
    _, ex = torch.frexp(bm)
    return torch.where(bm > 0, (ex - 1 - 14).clamp(-127, 127), torch.zeros_like(ex)).float()


def _round(Y, mistake=None):
    s = _exponents(Y)
    x = Y * torch.repeat_interleave(torch.exp2(-s), 32, 1)
    h = x.half().float()
    if mistake == "toward_zero":
        h = torch.where(h.abs() > x.abs(), torch.nextafter(h.half(), torch.zeros_like(h).half()).float(), h)
    if mistake == "neighbour_scale":
        s = torch.roll(s, 1, dims=1)
    return h * torch.repeat_interleave(torch.exp2(s), 32, 1)


def test_specified_rounding_within_bound():
    for seed in range(3):
        yp, A, inv, w = _case(seed)
        y_step = _combine(yp, inv, w)
        bound = scaled16_bound(yp, A, inv, w, y_step)
        assert bool(((_combine(_round(yp), inv, w) - y_step).abs().double() <= bound).all())


def test_planted_mistakes_break_bound():
    yp, A, inv, w = _case(0)
    y_step = _combine(yp, inv, w)
    bound = scaled16_bound(yp, A, inv, w, y_step)
    coarse = 2.0 ** -10 * float(yp[:A].abs().max())
    for mistake in ("toward_zero", "neighbour_scale"):
        d = (_combine(_round(yp, mistake), inv, w) - y_step).abs().double()
        assert not bool((d <= bound).all()), mistake
    d = (_combine(_round(yp, "toward_zero"), inv, w) - y_step).abs().double()
    assert bool((d <= coarse).all())  # the coarse bound alone would not see it
