"""Seeded synthetic inputs shaped like the workloads on the pages.

This module only draws random tensors and routing tables; it holds none of the
method's arithmetic (no rotation, scaling, rounding or GEMM), so both the
oracle and the HIP path can be fed from it.  Every tensor comes from a torch
Generator seeded explicitly; the same bf16 tensor is handed to both sides.

The pages train Dense 1.5B, MoE 7.9B and MoE 124B models (UFP4 abstract) and
note that training tensors carry outlier coordinates (UFP4 summary, Method);
the 2D-block page trains OLMo-1B/7B and a 30B MoE.  No dataset or checkpoint
is used: these tensors stand in for the pretraining activations, weights and
output gradients of one linear layer.
"""
from dataclasses import dataclass, field
from typing import List, Optional

import torch

E1M2, INT4, E2M1 = 0, 1, 2
RTNE, SR = 0, 1
SCALE_F32, SCALE_POW2 = 0, 1


def _gen(seed, device):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def normal_bf16(shape, std, seed, device="cpu"):
    g = _gen(seed, device)
    x = torch.randn(*shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x.to(torch.bfloat16)


def student_t_bf16(shape, nu, seed, device="cpu"):
    """Student-t(nu) for integer nu: Z / sqrt(chi2_nu / nu)."""
    g = _gen(seed, device)
    z = torch.randn(*shape, generator=g, device=device, dtype=torch.float32)
    chi = torch.zeros(shape, device=device, dtype=torch.float32)
    for _ in range(int(nu)):
        w = torch.randn(*shape, generator=g, device=device, dtype=torch.float32)
        chi.addcmul_(w, w)
    return (z / torch.sqrt(chi / nu)).to(torch.bfloat16)


def scale_channels(x, frac, factor, seed):
    """Multiply a seeded random set of round(frac * cols) columns by factor."""
    cols = x.shape[-1]
    nsel = max(1, int(round(frac * cols)))
    g = _gen(seed, "cpu")
    idx = torch.randperm(cols, generator=g)[:nsel].to(x.device)
    y = x.float()
    y[..., idx] *= factor
    return y.to(torch.bfloat16), idx.cpu()


def scale_elements(x, frac, factor, seed):
    """Multiply a seeded Bernoulli(frac) mask of entries by factor."""
    g = _gen(seed, x.device.type)
    mask = torch.rand(x.shape, generator=g, device=x.device) < frac
    y = x.float()
    y[mask] *= factor
    return y.to(torch.bfloat16)


def round_up(v, m):
    return ((int(v) + m - 1) // m) * m


def topk_routing(tokens, experts, k, weights, seed):
    """Each token picks k distinct experts by Gumbel-top-k over log weights.
    Returns (expert ids [tokens, k], tokens per expert)."""
    g = _gen(seed, "cpu")
    logits = torch.log(torch.as_tensor(weights, dtype=torch.float64)).expand(tokens, experts)
    u = torch.rand(tokens, experts, generator=g, dtype=torch.float64).clamp_(1e-300, 1.0)
    gumbel = -torch.log(-torch.log(u))
    ids = torch.topk(logits + gumbel, k, dim=1).indices
    counts = torch.bincount(ids.reshape(-1), minlength=experts)
    return ids, counts


def zipf_weights(experts, alpha, seed):
    """Zipf(alpha) popularity over a seeded random ranking of the experts."""
    g = _gen(seed, "cpu")
    rank = torch.randperm(experts, generator=g).to(torch.float64) + 1.0
    return rank.pow(-alpha)


def permute_by_expert(ids, counts, pad_to):
    """Token gather order grouped by expert, each expert padded to a multiple
    of pad_to rows.  Returns (gather index with -1 for padding rows,
    padded offsets [E+1], unpadded counts)."""
    tokens, k = ids.shape
    flat = ids.reshape(-1)
    order = torch.argsort(flat, stable=True)
    token_of = order // k
    rows: List[torch.Tensor] = []
    offsets = [0]
    start = 0
    for e in range(counts.numel()):
        c = int(counts[e])
        seg = token_of[start:start + c]
        start += c
        padded = round_up(c, pad_to) if c else 0
        if padded > c:
            seg = torch.cat([seg, torch.full((padded - c,), -1, dtype=seg.dtype)])
        rows.append(seg)
        offsets.append(offsets[-1] + padded)
    return torch.cat(rows), torch.tensor(offsets, dtype=torch.int64), counts.clone()


def gather_rows(x, gather):
    """x[gather] with zero rows where gather == -1."""
    out = torch.zeros((gather.numel(), x.shape[1]), dtype=x.dtype, device=x.device)
    valid = gather >= 0
    g = gather.to(x.device)
    vd = valid.to(x.device)
    out[vd] = x[g[vd]]
    return out


@dataclass
class QuantParams:
    """Parameters of one quantization call, as plain numbers."""
    grid: int
    rounding: int
    scale_mode: int
    block_rows: int
    block_cols: int
    rht_n: int
    sign_seed: int
    sr_seed: int = 0
    sr_stream: int = 0


@dataclass
class Workload:
    name: str
    tensors: dict = field(default_factory=dict)
    meta: dict = field(default_factory=dict)


def config1(device="cpu"):
    """FPROP only: X, W 256 x 256 N(0,1); n = 16, 1 x 16 fp32 scales, E1M2, RTNE."""
    g = _gen(0, device)
    X = torch.randn(256, 256, generator=g, device=device).to(torch.bfloat16)
    W = torch.randn(256, 256, generator=g, device=device).to(torch.bfloat16)
    q = QuantParams(E1M2, RTNE, SCALE_F32, 1, 16, 16, sign_seed=0)
    return Workload("fprop 256x256x256 E1M2 n16 b16", {"X": X, "W": W}, {"q": q})


def config2(device="cpu", M=8192, K=2048, N=8192):
    """Dense linear layer: X [M,K] N(0,1) with 0.5% channels x50, W [N,K]
    N(0,0.02), dY [M,N] N(0,1e-3); n = 16 on every GEMM's K, 1 x 16 blocks."""
    X = normal_bf16((M, K), 1.0, 2001, device)
    X, ch = scale_channels(X, 0.005, 50.0, 2002)
    W = normal_bf16((N, K), 0.02, 2003, device)
    dY = normal_bf16((M, N), 1e-3, 2004, device)
    return Workload(f"dense linear M{M} K{K} N{N}", {"X": X, "W": W, "dY": dY},
                    {"outlier_channels": ch, "sign_seeds": (2101, 2102, 2103), "sr_seed": 2201,
                     "n": 16, "b": 16})


def config3(device="cpu", tokens=16384, experts=64, hidden=2048, ffn=1408, topk=6):
    """MoE: Zipf(1.1) top-6 routing, Student-t(4) activations, n = 32, 1 x 32."""
    w = zipf_weights(experts, 1.1, 3000)
    ids, counts = topk_routing(tokens, experts, topk, w, 3000)
    gather, offsets, counts = permute_by_expert(ids, counts, 32)
    X = student_t_bf16((tokens, hidden), 4, 3001, device)
    W = normal_bf16((experts * ffn, hidden), 0.02, 3003, device)
    dY = normal_bf16((int(offsets[-1]), ffn), 1e-3, 3004, device)
    dY = dY * (gather >= 0).to(device).unsqueeze(1).to(dY.dtype)
    return Workload("moe64 h2048 f1408 top6 zipf1.1",
                    {"X": X, "W": W, "dY_perm": dY},
                    {"gather": gather, "offsets": offsets, "counts": counts, "experts": experts,
                     "hidden": hidden, "ffn": ffn, "sign_seeds": (3101, 3102, 3103),
                     "sr_seed": 3201, "n": 32, "b": 32})


def config4(device="cpu", tokens=32768, experts=16, hidden=5120, ffn=1536, topk=8):
    """Large-MoE share: uniform top-8 of 16, n = 128, 1 x 16, INT4."""
    w = torch.ones(experts, dtype=torch.float64)
    ids, counts = topk_routing(tokens, experts, topk, w, 4000)
    gather, offsets, counts = permute_by_expert(ids, counts, 128)
    X = normal_bf16((tokens, hidden), 1.0, 4001, device)
    X = scale_elements(X, 0.001, 100.0, 4002)
    W = normal_bf16((experts * ffn, hidden), 0.02, 4003, device)
    dY = normal_bf16((int(offsets[-1]), ffn), 1e-3, 4004, device)
    dY = dY * (gather >= 0).to(device).unsqueeze(1).to(dY.dtype)
    return Workload("moe16-share h5120 f1536 top8 uniform",
                    {"X": X, "W": W, "dY_perm": dY},
                    {"gather": gather, "offsets": offsets, "counts": counts, "experts": experts,
                     "hidden": hidden, "ffn": ffn, "sign_seeds": (4101, 4102, 4103),
                     "sr_seed": 4201, "n": 128, "b": 16})


def config5(device="cpu", M=16384, K=4096, N=4096):
    """2D square blocks 32 x 32, power-of-two scales, SR, no rotation."""
    X = normal_bf16((M, K), 1.0, 5001, device)
    W = normal_bf16((N, K), 1.0, 5002, device)
    dY = normal_bf16((M, N), 1e-3, 5003, device)
    return Workload(f"2d-block M{M} K{K} N{N}", {"X": X, "W": W, "dY": dY},
                    {"sr_seed": 5201, "b": 32})


def bits(x):
    """bf16 tensor -> uint16 numpy bits (host copy)."""
    return x.detach().contiguous().cpu().view(torch.int16).numpy().view("uint16")
