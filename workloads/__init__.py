"""Seeded synthetic inputs for the LatentMoE layer.

This module only draws random numbers and lays them out; it holds none of the
layer's arithmetic.  Both the CPU oracle (``oracle/``) and the HIP path consume
what it returns, so it is the single source of inputs for parity tests and the
bench.

Shapes follow the LatentMoE feed-forward of Kimi K3 as described by the
TokenSpeed AgentX post ("Model architecture": 16 of 896 routed experts plus two
shared experts) and the vLLM Kimi K3 post (section 1, "LatentMoE: Dimensionality
Reduction at the Routing Inlet, Restoration at the Outlet": 512 -> 256 latent
example).

Every tensor gets its own torch generator seeded from (seed, tensor name), so a
tensor does not change when another one is added or resized.  ``device`` picks
the generator: the CPU and GPU generators give different (but each
deterministic) values; a test always hands the same tensors to both sides.

Weight layout is ``[out, in]`` (reduction dim contiguous):
  w_in [l,d]; w1, w3 [E,I,l]; w2 [E,l,I]; w_out [d,l]; w_r [E,l] (router gate);
  ws1, ws3 [S,Is,d]; ws2 [S,d,Is]; norm_w [l].
MXFP4 experts: codes packed two per byte (even K index in the low nibble)
  w1q, w3q [E,I,l/2] u8 with e8m0 scales s1, s3 [E,I,l/32];
  w2q [E,l,I/2] u8 with s2 [E,l,I/32].
"""
from __future__ import annotations

import dataclasses
import hashlib
from typing import Optional

import torch

BF16 = torch.bfloat16


@dataclasses.dataclass(frozen=True)
class LayerConfig:
    name: str
    T: int            # tokens (rows in rows mode)
    d: int            # hidden width (0 in rows mode)
    l: int            # latent width
    E: int            # routed experts (local experts in rows mode)
    k: int            # experts per token (1 in rows mode)
    S: int            # shared experts
    I: int            # routed SwiGLU intermediate
    Is: int           # shared SwiGLU intermediate
    rows_mode: bool = False   # expert-parallel share: ids + weights given, no projections
    mxfp4: bool = False       # routed expert weights in MXFP4
    w4a16: bool = False       # with mxfp4: bf16 activations (else MXFP8 activations, w4a8)
    router_gemm: bool = False # logits computed from the latent by a gate w_r [E,l] (else given)
    norm: bool = True         # routed-latent RMSNorm with gain 1
    eps: float = 1e-6
    zipf_s: float = 0.0       # rows mode: Zipf exponent of the expert load
    seed: int = 0
    os: bool = False          # run through the output-stationary layer call (same inputs)


CONFIGS = {
    # 64 tokens, d=512 -> latent 256, 16 experts top-4, one shared expert, I=128
    "tiny": LayerConfig("tiny", T=64, d=512, l=256, E=16, k=4, S=1, I=128, Is=128),
    # decode batch of 256 tokens, 512 -> 256 latent, 896 experts top-16 + 2 shared, I=256
    "decode": LayerConfig("decode", T=256, d=512, l=256, E=896, k=16, S=2, I=256, Is=256),
    # prefill: 8192 tokens, 7168 -> 2048 latent, 896 experts top-16 + 2 shared, I=512
    "prefill": LayerConfig("prefill", T=8192, d=7168, l=2048, E=896, k=16, S=2, I=512, Is=512),
    # one expert-parallel rank's share: 56 local experts, 16384 received rows, Zipf(1.1) load
    "ep_share": LayerConfig("ep_share", T=16384, d=0, l=2048, E=56, k=1, S=0, I=512, Is=0,
                            rows_mode=True, norm=False, zipf_s=1.1),
    # prefill shape at 16384 tokens with MXFP4 routed experts
    "prefill_mxfp4": LayerConfig("prefill_mxfp4", T=16384, d=7168, l=2048, E=896, k=16, S=2,
                                 I=512, Is=512, mxfp4=True),
    # the 16384-token prefill shape with bf16 routed experts (~293 rows per expert)
    "prefill_bf16_16k": LayerConfig("prefill_bf16_16k", T=16384, d=7168, l=2048, E=896, k=16, S=2,
                                    I=512, Is=512),
    # the 16384-token prefill shape with MXFP4 routed experts and bf16 activations (w4a16)
    "prefill_w4a16": LayerConfig("prefill_w4a16", T=16384, d=7168, l=2048, E=896, k=16, S=2,
                                 I=512, Is=512, mxfp4=True, w4a16=True),
    # the decode batch with MXFP4 routed experts and bf16 activations (w4a16)
    "decode_w4a16": LayerConfig("decode_w4a16", T=256, d=512, l=256, E=896, k=16, S=2, I=256, Is=256,
                                mxfp4=True, w4a16=True),
    # the decode batches through the output-stationary layer call (no permutation)
    "decode_os": LayerConfig("decode_os", T=256, d=512, l=256, E=896, k=16, S=2, I=256, Is=256, os=True),
    "decode_w4a16_os": LayerConfig("decode_w4a16_os", T=256, d=512, l=256, E=896, k=16, S=2, I=256, Is=256,
                                   mxfp4=True, w4a16=True, os=True),
    # the decode shape with the router's logits computed from the latent (gate [E,l])
    "decode_gate": LayerConfig("decode_gate", T=256, d=512, l=256, E=896, k=16, S=2, I=256, Is=256,
                               router_gemm=True),
}


def _gen(seed: int, name: str, device) -> torch.Generator:
    h = hashlib.sha256(f"{seed}:{name}".encode()).digest()
    g = torch.Generator(device=device)
    g.manual_seed(int.from_bytes(h[:8], "little") & ((1 << 63) - 1))
    return g


def normal_bf16(seed, name, shape, std, device="cpu", mean=0.0) -> torch.Tensor:
    """N(mean, std) drawn in fp32, stored as bf16 (round-to-nearest-even cast)."""
    g = _gen(seed, name, device)
    t = torch.randn(*shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    if mean != 0.0:
        t.add_(mean)
    return t.to(BF16)


def router_gate_std(d: int, l: int) -> float:
    """Std of the router gate's entries that gives logits of unit variance when
    x ~ N(0,1) and w_in ~ N(0, 0.02) (the latent then has variance d * 0.02^2)."""
    return 1.0 / (l * d * 0.02 ** 2) ** 0.5


def grid_bf16(seed, name, shape, levels: int, step: float, device="cpu") -> torch.Tensor:
    """Integers drawn uniformly from [-levels, levels], times ``step`` (a power of
    two), stored as bf16: values on a coarse grid, so that sums of their
    products are exact in fp32 while the magnitudes stay small."""
    g = _gen(seed, name, device)
    t = torch.randint(-levels, levels + 1, tuple(shape), generator=g, device=device, dtype=torch.int32)
    return (t.to(torch.float32) * step).to(BF16)


def separated_logits(seed, name, T, E, k, device="cpu", min_gap=1e-3) -> torch.Tensor:
    """fp32 N(0,1) router logits, each token redrawn until the k+1 largest values
    are pairwise at least ``min_gap`` apart (so top-k is unambiguous)."""
    g = _gen(seed, name, device)
    out = torch.randn(T, E, generator=g, device=device, dtype=torch.float32)
    kk = min(k + 1, E)
    for _ in range(1000):
        top = torch.topk(out, kk, dim=1).values
        bad = (top[:, :-1] - top[:, 1:] < min_gap).any(dim=1) if kk > 1 else \
            torch.zeros(T, dtype=torch.bool, device=device)
        nbad = int(bad.sum())
        if nbad == 0:
            return out
        out[bad] = torch.randn(nbad, E, generator=g, device=device, dtype=torch.float32)
    raise RuntimeError("could not draw separated logits")


def zipf_ids(seed, name, R, E, s, device="cpu") -> torch.Tensor:
    """R i.i.d. expert ids whose load follows Zipf(s) over ranks 1..E; the rank ->
    expert id map is a seeded permutation."""
    g = _gen(seed, name, "cpu")
    ranks = torch.arange(1, E + 1, dtype=torch.float64)
    p = ranks.pow(-s)
    p /= p.sum()
    draws = torch.multinomial(p, R, replacement=True, generator=g)
    perm = torch.randperm(E, generator=g)
    return perm[draws].to(torch.int32).to(device)


def uniform_weights(seed, name, shape, device="cpu") -> torch.Tensor:
    """fp32 combine weights drawn from U(0, 1]."""
    g = _gen(seed, name, device)
    u = torch.rand(*shape, generator=g, device=device, dtype=torch.float32)
    return 1.0 - u


# Magnitude distribution of the MXFP4 element codes drawn below.  The codes
# 0..7 are the non-negative e2m1 encodings; the probabilities roughly follow a
# Gaussian block scaled so its max lands near the top code.  They are input
# structure only (no encoder is involved).
_E2M1_CODE_PROBS = [0.08, 0.15, 0.15, 0.14, 0.13, 0.20, 0.10, 0.05]


def mxfp4_weights(seed, name, E, N, K, device="cpu"):
    """Random MXFP4 weight matrix [E,N,K]: packed e2m1 codes [E,N,K/2] (even K in
    the low nibble) and e8m0 scales [E,N,K/32] around 2^-7 (codes 119..121), so
    the dequantised values have a spread near N(0, 0.02).  Codes are drawn by
    inverting the categorical CDF on uniform draws, in chunks."""
    assert K % 32 == 0
    cdf = torch.tensor(_E2M1_CODE_PROBS, dtype=torch.float64).cumsum(0)
    cdf = (cdf / cdf[-1]).to(torch.float32).to(device)
    g = _gen(seed, name + ".codes", device)
    nbytes = E * N * K // 2
    packed = torch.empty(nbytes, dtype=torch.uint8, device=device)
    chunk = 1 << 25
    for b0 in range(0, nbytes, chunk):
        n = min(chunk, nbytes - b0)
        u = torch.rand(2 * n, generator=g, device=device)
        mag = torch.searchsorted(cdf, u, right=True).clamp_(max=7).to(torch.uint8)
        sign = (torch.rand(2 * n, generator=g, device=device) < 0.5).to(torch.uint8) << 3
        codes = (mag | sign).view(n, 2)
        packed[b0:b0 + n] = codes[:, 0] | (codes[:, 1] << 4)
    gs = _gen(seed, name + ".scales", device)
    scdf = torch.tensor([0.25, 0.75], dtype=torch.float32, device=device)
    us = torch.rand(E * N * (K // 32), generator=gs, device=device)
    scales = (119 + torch.searchsorted(scdf, us, right=True)).to(torch.uint8)
    return packed.view(E, N, K // 2), scales.view(E, N, K // 32)


def make_inputs(cfg: LayerConfig, device="cpu", norm_w: Optional[str] = None) -> dict:
    """All inputs of one layer call for ``cfg``.

    norm_w: None -> the config's default (ones if cfg.norm else absent),
            "ones", "random" (N(1, 0.1)) or "none".
    """
    s = cfg.seed
    inp = {"cfg": cfg}
    if cfg.rows_mode:
        inp["x"] = normal_bf16(s, "x", (cfg.T, cfg.l), 1.0, device)
        inp["ids"] = zipf_ids(s, "ids", cfg.T, cfg.E, cfg.zipf_s, device).view(cfg.T, 1)
        inp["weights"] = uniform_weights(s, "weights", (cfg.T, 1), device)
    else:
        inp["x"] = normal_bf16(s, "x", (cfg.T, cfg.d), 1.0, device)
        if cfg.router_gemm:
            # gate on the latent, scaled so that the logits are about N(0,1)
            # (z = x w_in^T has variance d * 0.02^2)
            inp["w_r"] = normal_bf16(s, "w_r", (cfg.E, cfg.l), router_gate_std(cfg.d, cfg.l), device)
        else:
            inp["logits"] = separated_logits(s, "logits", cfg.T, cfg.E, cfg.k, device)
        inp["w_in"] = normal_bf16(s, "w_in", (cfg.l, cfg.d), 0.02, device)
        inp["w_out"] = normal_bf16(s, "w_out", (cfg.d, cfg.l), 0.02, device)
        if cfg.S > 0:
            inp["ws1"] = normal_bf16(s, "ws1", (cfg.S, cfg.Is, cfg.d), 0.02, device)
            inp["ws3"] = normal_bf16(s, "ws3", (cfg.S, cfg.Is, cfg.d), 0.02, device)
            inp["ws2"] = normal_bf16(s, "ws2", (cfg.S, cfg.d, cfg.Is), 0.02, device)
    if cfg.mxfp4:
        inp["w1q"], inp["s1"] = mxfp4_weights(s, "w1", cfg.E, cfg.I, cfg.l, device)
        inp["w3q"], inp["s3"] = mxfp4_weights(s, "w3", cfg.E, cfg.I, cfg.l, device)
        inp["w2q"], inp["s2"] = mxfp4_weights(s, "w2", cfg.E, cfg.l, cfg.I, device)
    else:
        inp["w1"] = normal_bf16(s, "w1", (cfg.E, cfg.I, cfg.l), 0.02, device)
        inp["w3"] = normal_bf16(s, "w3", (cfg.E, cfg.I, cfg.l), 0.02, device)
        inp["w2"] = normal_bf16(s, "w2", (cfg.E, cfg.l, cfg.I), 0.02, device)
    mode = norm_w or ("ones" if cfg.norm else "none")
    if mode == "ones":
        inp["norm_w"] = torch.ones(cfg.l, dtype=BF16, device=device)
    elif mode == "random":
        inp["norm_w"] = normal_bf16(s, "norm_w", (cfg.l,), 0.1, device, mean=1.0)
    elif mode != "none":
        raise ValueError(mode)
    return inp


def custom(name="custom", **kw) -> LayerConfig:
    """A LayerConfig with explicit fields (for ragged and edge-case tests)."""
    return LayerConfig(name=name, **kw)
