"""Seeded synthetic inputs for the Q8_0 matmul workloads.

This module only draws numbers: fp32 weights and activations, routing lists
and outlier channels.  It holds none of the method's arithmetic (no
quantization, no dot products); both the GPU path and the CPU oracle take
their inputs from here.

Recipe: every tensor has its own torch.Generator seeded with a 63-bit hash of
(base seed, workload, tensor name, index), so any tensor (e.g. one expert's
matrix) can be regenerated alone.  Values are torch.randn * std in fp32 on the
requested device (CUDA Philox on the GPU, the CPU generator on the host: the
two devices give different but individually reproducible draws).  Routing and
outlier-channel choices are always drawn on the CPU.

Workloads follow the ds4 layer shapes given on the pages ("Part 3: 模型架构",
section 1, the layer weight table; GGUF [in, out] notation):
  tiny       W [128 x 256], x [4 x 256]; one all-zero block and one x50 outlier
             on each side.
  attn_q_b   decode: in 1024 -> out 32768 (64 heads x 512), n_tok 1.
  decode5    decode: attn_q_a 4096->1024, attn_kv 4096->512,
             attn_output_a 32768->1024, attn_output_b 1024->4096,
             ffn_gate_inp 4096->256, each n_tok 1 with its own x.
  moe        256 experts x {gate, up: 4096->2048; down: 2048->4096} + one
             shared expert; 64 tokens, 8 distinct experts per token drawn
             uniformly; down input `mid` [64*8 + 64 rows x 2048] ~ N(0, 1).
  prefill_a  shared-expert gate 4096->2048 at n_tok 4096.
  prefill_b  attn_output_a 32768->1024 at n_tok 2048.
Weights ~ N(0, 0.02), activations ~ N(0, 1); prefill activations have 1% of
their input channels (chosen without replacement) multiplied by 20.
"""
from __future__ import annotations

import hashlib

import torch

BASE_SEED = 0
W_STD = 0.02
X_STD = 1.0

DECODE5 = [  # name, in_dim, out_dim
    ("attn_q_a", 4096, 1024),
    ("attn_kv", 4096, 512),
    ("attn_output_a", 32768, 1024),
    ("attn_output_b", 1024, 4096),
    ("ffn_gate_inp", 4096, 256),
]

MOE = dict(n_expert=256, n_used=8, n_tok=64, d_model=4096, d_ff=2048)

PREFILL = {
    "prefill_a": dict(in_dim=4096, out_dim=2048, n_tok=4096),
    "prefill_b": dict(in_dim=32768, out_dim=1024, n_tok=2048),
}


def seed_of(*parts) -> int:
    key = "|".join(str(p) for p in (BASE_SEED,) + parts).encode()
    return int.from_bytes(hashlib.blake2b(key, digest_size=8).digest(), "little") >> 1


def _gen(device, *parts) -> torch.Generator:
    g = torch.Generator(device=torch.device(device))
    g.manual_seed(seed_of(*parts))
    return g


def normal(shape, std, device, *parts) -> torch.Tensor:
    g = _gen(device, *parts)
    t = torch.randn(*shape, generator=g, device=device, dtype=torch.float32)
    return t.mul_(std) if std != 1.0 else t


def tiny(device="cpu"):
    w = normal((128, 256), W_STD, device, "tiny", "w")
    x = normal((4, 256), X_STD, device, "tiny", "x")
    x[0, 0:32] = 0.0           # all-zero block: token 0, block 0
    w[0, 5 * 32:6 * 32] = 0.0  # all-zero block: row 0, block 5
    x[1, 3 * 32 + 7] *= 50.0   # single x50 outlier: token 1, block 3
    w[1, 2 * 32 + 0] *= 50.0   # single x50 outlier: row 1, block 2
    return dict(w=w, x=x, in_dim=256, out_dim=128, n_tok=4)


def attn_q_b(device="cpu", copy=0):
    w = normal((32768, 1024), W_STD, device, "attn_q_b", "w", copy)
    x = normal((1, 1024), X_STD, device, "attn_q_b", "x")
    return dict(w=w, x=x, in_dim=1024, out_dim=32768, n_tok=1)


def decode5(device="cpu", copy=0):
    out = []
    for name, k, n in DECODE5:
        out.append(dict(name=name, in_dim=k, out_dim=n, n_tok=1,
                        w=normal((n, k), W_STD, device, "decode5", name, "w", copy),
                        x=normal((1, k), X_STD, device, "decode5", name, "x")))
    return out


def moe_routing() -> torch.Tensor:
    """int32 [64][8]: 8 distinct experts per token, uniform, drawn on the CPU."""
    g = _gen("cpu", "moe", "route")
    rows = [torch.randperm(MOE["n_expert"], generator=g)[:MOE["n_used"]]
            for _ in range(MOE["n_tok"])]
    return torch.stack(rows).to(torch.int32)


def moe_expert(e: int, which: str, device="cpu") -> torch.Tensor:
    """fp32 weights of routed expert e (0..255) or the shared expert (e = -1)."""
    d, f = MOE["d_model"], MOE["d_ff"]
    shape = (f, d) if which in ("gate", "up") else (d, f)
    tag = "shared" if e < 0 else "expert"
    return normal(shape, W_STD, device, "moe", tag, e, which)


def moe_acts(device="cpu"):
    n_pairs = MOE["n_tok"] * MOE["n_used"]
    x = normal((MOE["n_tok"], MOE["d_model"]), X_STD, device, "moe", "x")
    mid = normal((n_pairs + MOE["n_tok"], MOE["d_ff"]), X_STD, device, "moe", "mid")
    return x, mid


def outlier_channels(name: str, in_dim: int) -> torch.Tensor:
    g = _gen("cpu", name, "outlier_channels")
    n = in_dim // 100
    return torch.sort(torch.randperm(in_dim, generator=g)[:n]).values


def prefill(name: str, device="cpu", rows=None, tokens=None):
    """Prefill workload; rows/tokens restrict to the first rows/tokens drawn
    (the full tensors are drawn and sliced, so slices match the full draw)."""
    cfg = PREFILL[name]
    w = normal((cfg["out_dim"], cfg["in_dim"]), W_STD, device, name, "w")
    x = normal((cfg["n_tok"], cfg["in_dim"]), X_STD, device, name, "x")
    ch = outlier_channels(name, cfg["in_dim"]).to(x.device)
    x[:, ch] *= 20.0
    if rows is not None:
        w = w[:rows].contiguous()
    if tokens is not None:
        x = x[:tokens].contiguous()
    return dict(w=w, x=x, **cfg)
