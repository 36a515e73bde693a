"""Seeded synthetic inputs drawn directly on the GPU with torch generators (for the
benchmark's large workloads, up to a whole 64-layer 32B-class policy).  Same
distributions as the numpy generators in this package: N(0, std) with optional
outlier input channels, Student-t(3) activations, rank-64 updates; values are drawn
in float32 and rounded to bf16.  No step of the method lives here."""
import torch


def gen(seed, device="cuda"):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def seed_of(cfg, shape_idx, role, layer=0, step=0):
    return (((cfg * 131 + shape_idx) * 131 + role) * 1031 + layer) * 1031 + step


def normal_bf16(shape, std, g, outlier_frac=0.0, outlier_mult=1.0, device="cuda"):
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    x.mul_(std)
    if outlier_frac > 0:
        k = shape[-1]
        cnt = int(round(outlier_frac * k))
        cols = torch.randperm(k, generator=g, device=device)[:cnt]
        x[..., cols] *= outlier_mult
    return x.to(torch.bfloat16)


def student_t_bf16(shape, nu, g, device="cuda"):
    z = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    chi2 = torch.zeros(shape, device=device, dtype=torch.float32)
    for _ in range(int(nu)):
        e = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        chi2.addcmul_(e, e)
    return (z / torch.sqrt(chi2 / nu)).to(torch.bfloat16)


def rank_update_(w, rank, std, g):
    """w <- bf16(fp32(w) + (std / sqrt(rank)) * B A), A [rank, K], B [N, rank] ~ N(0, 1),
    so each entry of the update has standard deviation `std`."""
    n, k = w.shape
    a = torch.randn((rank, k), generator=g, device=w.device, dtype=torch.float32)
    b = torch.randn((n, rank), generator=g, device=w.device, dtype=torch.float32)
    upd = (b @ a).mul_(std / rank ** 0.5)
    w.copy_((w.float() + upd).to(torch.bfloat16))
