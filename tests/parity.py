"""Helpers shared by the parity tests (comparison metrics, input staging)."""
import sys

import torch

NAN_BF16 = 0x7FC0


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def metrics(got, ref):
    """Tolerance metrics.

    rel_i = |g_i - o_i| / max(|o_i|, rms(o)): an element at or above the
    output's RMS is judged against itself, a smaller one against the RMS.
    Both implementations store z, H, Y, rhat and hs in bf16, and fp32
    summation order flips some of those roundings by one ulp on either side;
    the flips reach every output with an absolute size of a fraction of a
    percent of the RMS, so a per-element ratio without a floor would be noise
    on near-zero outputs.  Also returned: MAE and ||g - o||_inf / ||o||_inf.
    """
    got, ref = got.double().cpu(), ref.double().cpu()
    floor = ref.pow(2).mean().sqrt().clamp_min(1e-30)
    diff = (got - ref).abs()
    rel = diff / torch.maximum(ref.abs(), floor)
    return {
        "max_rel": rel.max().item() if rel.numel() else 0.0,
        "mae": diff.mean().item() if diff.numel() else 0.0,
        "inf_ratio": (diff.max() / ref.abs().max().clamp_min(1e-30)).item() if diff.numel() else 0.0,
        "nan": bool(torch.isnan(got).any()),
    }


def assert_parity(got, ref, max_rel=2e-2, mae=1e-3, what="y"):
    m = metrics(got, ref)
    log(f"  {what}: max_rel={m['max_rel']:.3e} mae={m['mae']:.3e} inf_ratio={m['inf_ratio']:.3e}")
    assert not m["nan"], f"{what}: NaN in GPU output"
    assert m["max_rel"] <= max_rel, f"{what}: max_rel {m['max_rel']:.3e} > {max_rel}"
    assert m["mae"] <= mae, f"{what}: MAE {m['mae']:.3e} > {mae}"
    return m


def to_device(inp, device="cuda"):
    out = {}
    for k, v in inp.items():
        out[k] = v.to(device) if isinstance(v, torch.Tensor) else v
    return out


def to_host(inp):
    return to_device(inp, "cpu")


def poison_(t: torch.Tensor):
    """Fill a buffer with bf16 NaN patterns so that any unwritten read shows up."""
    if t.dtype == torch.uint8:
        t.view(torch.uint8).copy_(torch.tensor([0xC0, 0x7F], dtype=torch.uint8, device=t.device)
                                  .repeat(t.numel() // 2 + 1)[: t.numel()])
    else:
        t.view(torch.int16).fill_(NAN_BF16)
    return t


def assert_rowwise(got, ref, max_row_rel=5e-2, mae=5e-3, what="y"):
    """Block-quantised (MXFP4 w4a8) outputs: every token row within max_row_rel
    relative L2 error, and the global MAE bound.  One-ulp bf16 differences in
    the activations feeding the MXFP8 quantiser can move an e4m3 code by one
    step (1/8 relative) or a block's shared exponent, so single elements are
    compared through their row rather than one by one."""
    g, o = got.double().cpu(), ref.double().cpu()
    row_err = (g - o).norm(dim=1) / o.norm(dim=1).clamp_min(1e-30)
    m = metrics(got, ref)
    log(f"  {what}: max_row_rel={row_err.max().item():.3e} mae={m['mae']:.3e} "
        f"elementwise max_rel={m['max_rel']:.3e} inf_ratio={m['inf_ratio']:.3e}")
    assert not m["nan"], f"{what}: NaN in GPU output"
    assert row_err.max().item() <= max_row_rel, f"{what}: max row error {row_err.max().item():.3e}"
    assert m["mae"] <= mae, f"{what}: MAE {m['mae']:.3e} > {mae}"
    return m
