"""GPU parity at the edges of the number formats (rows mode, where the expert
GEMMs' input is the given x, so each row's scale can be set on its own).

* MXFP8 quantisation of activations holding NaN, infinities and values near
  the top of bf16's range: codes and scales bit-exact against the oracle's
  quantiser (a NaN or infinity makes its 32-element block a NaN block), NaN
  reaching exactly the output rows it should, finite rows at the bar.
* MXFP4 weights whose e8m0 block scales span the code range: each expert's
  weight rows use codes from a window [c - 30, c], the windows of the experts
  together covering 0..254 (w4a8) or 2..252 (w4a16, where the weights are
  upcast to bf16 and must stay normal and finite there), and each expert's
  rows carry activations scaled so its outputs stay finite and normal.  Rows
  are compared expert by expert (their magnitudes differ by up to 2^200).
* Scale code 255 (e8m0 NaN) in one block: NaN in exactly the rows of that
  expert.
"""
import pytest
import torch

import oracle
import workloads as W
from tests.gpu_helpers import check_routing, run_gpu_layer
from tests.parity import W4A8_H_CODE_BUDGET, assert_mxfp8, elementwise_failures, log, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import latentmoe_expert_layer_amd  # noqa: F401
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    yield


def rows_cfg(name, R, E, l, I, w4a16, seed):
    return W.custom(name, T=R, d=0, l=l, E=E, k=1, S=0, I=I, Is=0, rows_mode=True, norm=False, zipf_s=0.5,
                    seed=seed, mxfp4=True, w4a16=w4a16)


def test_mxfp8_non_finite_and_large_activations():
    cfg = rows_cfg("mx_nonfinite", 600, 6, 256, 256, False, 21)
    inp = W.make_inputs(cfg)
    x = inp["x"].float()
    g = torch.Generator().manual_seed(4)
    x[5, 17] = float("nan")
    x[9, :] = float("nan")
    x[13, 40] = float("inf")
    x[14, 200] = float("-inf")
    x[20:40] = torch.randn(20, cfg.l, generator=g) * 1e17          # large, products stay finite
    x[41, 0:32] = torch.tensor([3.0e38, -3.0e38] * 16)              # one block at the top of bf16's range
    inp["x"] = x.to(torch.bfloat16)
    log(f"mxfp8 non-finite rows: {cfg}")
    r, y, views = run_gpu_layer(to_device(inp))
    check_routing(r, inp["ids"].view(-1), 1, cfg.E, weights=inp["weights"])
    ref = oracle.layer(inp, inp["ids"], inp["weights"], intermediates=True,
                       row_pos=oracle.permute(inp["ids"], cfg.E)[2])
    assert torch.equal(views["zq"].cpu(), ref["zq"]), "MXFP8 codes of the rows differ"
    assert torch.equal(views["zs"].cpu(), ref["zqs"]), "MXFP8 scales of the rows differ"
    zs = views["zs"].cpu()
    for row in (5, 9, 13, 14):
        assert int((zs[row] == 255).sum()) >= 1, row
    nan_rows = torch.isnan(ref["y"]).any(dim=1)
    assert torch.equal(torch.isnan(y.cpu()).any(dim=1), nan_rows), "NaN reaches other rows than the oracle's"
    assert bool(nan_rows[[5, 9, 13, 14]].all())
    big = torch.arange(20, 40)
    fails = elementwise_failures(y.cpu()[big], ref["y"][big], max_rel=5e-2, mae=1e-3, mae_rel=True,
                                 flip_budget=1e-3, what="large rows")
    assert not fails, fails
    ok = ~nan_rows
    ok[20:42] = False
    fails = elementwise_failures(y.cpu()[ok], ref["y"][ok], max_rel=5e-2, mae=1e-3, flip_budget=1e-3,
                                 what="other rows")
    assert not fails, fails


def set_scale_windows(inp, name, tops, width=30, seed=0):
    """Block scales of weight ``name`` (s1/s3/s2): expert e's codes uniform in
    [max(lo, tops[e] - width), tops[e]].  The e2m1 codes stay as drawn, except
    in blocks scaled by 2^126 or 2^127, where magnitudes above 1.5 are folded
    to 0..1.5 so that every dequantised weight is finite in fp32 (6 * 2^126
    is not)."""
    g = torch.Generator().manual_seed(seed)
    s = inp[name]
    for e, top in enumerate(tops):
        lo = max(0, top - width)
        s[e] = torch.randint(lo, top + 1, tuple(s[e].shape), generator=g, dtype=torch.int32).to(torch.uint8)
    q = inp[name.replace("s", "w") + "q"]                  # [E, N, K/2] packed codes
    big = (s >= 253).repeat_interleave(16, dim=-1)         # 16 bytes per 32-element block
    q[big] &= 0xBB                                         # keep sign and the two low bits of each code


def compare_by_expert(y, ref_y, ids, E, what, w4a8):
    bar = dict(max_rel=5e-2, flip_budget=1e-3) if w4a8 else dict(max_rel=2e-2)
    for e in range(E):
        rows = (ids.view(-1) == e).nonzero().flatten()
        if rows.numel() == 0:
            continue
        fails = elementwise_failures(y[rows], ref_y[rows], mae=1e-3, mae_rel=True, what=f"{what} expert {e}", **bar)
        assert not fails, fails


# the top codes of the experts' windows: together they cover [0, 254]
TOPS_W4A8 = [30, 60, 90, 120, 150, 180, 210, 240, 254]
# w4a16 upcasts to bf16: 0.5 * 2^(c-127) must be normal (c >= 2) and
# 6 * 2^(c-127) finite (c <= 252)
TOPS_W4A16 = [32, 60, 90, 120, 150, 180, 210, 240, 252]


@pytest.mark.parametrize("fmt", ["w4a8", "w4a16", "w4a16_tiled"])
@pytest.mark.parametrize("which", ["fc1", "fc2"])
def test_mxfp4_block_scales_across_the_code_range(fmt, which):
    w4a16 = fmt != "w4a8"
    tops = TOPS_W4A16 if w4a16 else TOPS_W4A8
    lo_code = 2 if w4a16 else 0
    E = len(tops)
    # w4a16: 280 rows (at most 32 per expert on average) run the weight-streaming
    # kernels, 900 rows the tiled ones
    rows = 280 if fmt == "w4a16" else 900
    cfg = rows_cfg(f"scales_{which}", rows, E, 256, 256, w4a16, 31 + (which == "fc2"))
    inp = W.make_inputs(cfg)
    ids = inp["ids"].view(-1).long()
    x = inp["x"].float()
    if which == "fc1":
        for n in ("s1", "s3"):
            set_scale_windows(inp, n, tops, seed=len(n) + (n == "s3"))
        inp["s1"].clamp_(min=lo_code)
        inp["s3"].clamp_(min=lo_code)
        # rows of expert e: x scaled by 2^(127 - top_e), kept within 2^+-100,
        # so z . w1 is O(1) where the scales allow
        sh = torch.tensor([float(min(100, max(-100, 127 - t))) for t in tops])
    else:
        set_scale_windows(inp, "s2", tops, seed=9)
        inp["s2"].clamp_(min=lo_code)
        # H ~ g^2 with g ~ 0.02 sqrt(l) |x|: aim H at 2^-(top_e - 127), kept
        # within 2^+-100 (normal in bf16), so that Y stays finite
        hexp = torch.tensor([float(min(100, max(-100, 127 - t))) for t in tops])
        sh = hexp / 2 - torch.log2(torch.tensor(0.02 * cfg.l ** 0.5))
    x = x * torch.pow(2.0, sh[ids]).view(-1, 1)
    inp["x"] = x.to(torch.bfloat16)
    codes = {n: torch.unique(inp[n]) for n in ("s1", "s3", "s2")}
    span = codes["s1" if which == "fc1" else "s2"]
    log(f"block scales {which} {'w4a16' if w4a16 else 'w4a8'}: codes {int(span.min())}..{int(span.max())} "
        f"({span.numel()} distinct)")
    assert int(span.min()) == lo_code and int(span.max()) == tops[-1]
    r, y, views = run_gpu_layer(to_device(inp))
    check_routing(r, inp["ids"].view(-1), 1, cfg.E, weights=inp["weights"])
    _, _, rp = oracle.permute(inp["ids"], cfg.E)
    ref = oracle.layer(inp, inp["ids"], inp["weights"], intermediates=True, row_pos=rp, act_quant=not w4a16)
    assert bool(torch.isfinite(ref["y"]).all()), "the oracle's outputs must stay finite here"
    yg = y.cpu()
    compare_by_expert(yg, ref["y"], ids, E, "y", not w4a16)
    pos = rp.long()
    compare_by_expert(views["Y"].cpu()[pos], ref["Y"][pos], ids, E, "Y", not w4a16)
    if not w4a16:
        assert_mxfp8(views["hq"].cpu(), views["hsc"].cpu(), ref["hq"], ref["hqs"], what="hq",
                     budget=W4A8_H_CODE_BUDGET)


@pytest.mark.parametrize("fmt", ["w4a8", "w4a16", "w4a16_tiled"])
def test_mxfp4_nan_block_scale(fmt):
    """e8m0 code 255 is NaN: one block of expert 2's W1 carries it, so exactly
    the rows routed to expert 2 come out NaN (w4a16: 150 rows over 5 experts
    run the weight-streaming kernels, 600 the tiled ones)."""
    w4a16 = fmt != "w4a8"
    cfg = rows_cfg("scale_nan", 150 if fmt == "w4a16" else (600 if w4a16 else 300), 5, 256, 256, w4a16, 41)
    inp = W.make_inputs(cfg)
    inp["s1"][2, 7, 3] = 255
    r, y, views = run_gpu_layer(to_device(inp))
    ids = inp["ids"].view(-1)
    ref = oracle.layer(inp, inp["ids"], inp["weights"], act_quant=not w4a16)["y"]
    want = ids == 2
    assert bool(want.any())
    assert torch.equal(torch.isnan(ref).any(dim=1), want)
    assert torch.equal(torch.isnan(y.cpu()).all(dim=1), want), "NaN rows differ from the rows of expert 2"
    fails = elementwise_failures(y.cpu()[~want], ref[~want], max_rel=5e-2 if not w4a16 else 2e-2, mae=1e-3,
                                 flip_budget=1e-3 if not w4a16 else 0.0, what="other rows")
    assert not fails, fails
