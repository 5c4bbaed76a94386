"""Helpers shared by the parity tests (comparison metrics, input staging).

The bars (a reading of the tolerance the layer is specified with):
 * bf16 path: every element within max relative error 2e-2, where an
   element's error is |g - o| / max(|o|, rms(o)), and mean absolute error
   1e-3 (intermediates: 1e-3 * rms(o), since their scale is not the
   output's).  Both sides store z, H, Y, rhat and hs in bf16 and sum in
   different fp32 orders, so some of those roundings land one ulp apart; the
   oracle evaluated in ascending and in descending K order disagrees by up to
   ~1.2e-2 under this floor but by up to ~9e-2 under a floor of 0.1 * rms(o)
   (tests/test_oracle_pins.py measures both), so the floor is rms(o).
 * MXFP4 w4a8 path: the same element-wise test at 5e-2, with a flip budget:
   at most a stated fraction of elements may exceed it, each by no more than
   W4A8_FLIP_MAX.  MXFP8 codes are compared through their values: at most a
   stated fraction may differ, each by about one e4m3 ulp (below).
 * Every bar holds per column and per row group (an expert's tile, a
   256-token tile) too, not only on average, so one wrong column or one
   wrong tile cannot hide in the mean.
"""
import sys

import torch

NAN_BF16 = 0x7FC0


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _rms(o):
    return o.pow(2).mean().sqrt().clamp_min(1e-30) if o.numel() else torch.tensor(1.0, dtype=torch.float64)


def metrics(got, ref):
    """rel_i = |g_i - o_i| / max(|o_i|, rms(o)) over the finite reference
    elements; also MAE and ||g - o||_inf / ||o||_inf."""
    got, ref = got.double().cpu(), ref.double().cpu()
    fin = torch.isfinite(ref)
    g, o = got[fin], ref[fin]
    floor = _rms(o)
    diff = (g - o).abs()
    rel = diff / torch.maximum(o.abs(), floor)
    return {
        "max_rel": rel.max().item() if rel.numel() else 0.0,
        "mae": diff.mean().item() if diff.numel() else 0.0,
        "rms": floor.item(),
        "inf_ratio": (diff.max() / o.abs().max().clamp_min(1e-30)).item() if diff.numel() else 0.0,
        "nan": bool(torch.isnan(got).any()),
    }


def elementwise_failures(got, ref, *, max_rel=2e-2, mae=1e-3, mae_rel=False, flip_budget=0.0,
                         flip_max=0.125, cols=True, groups=None, what="y"):
    """All reasons why ``got`` misses ``ref`` (an empty list = pass).

    got, ref: [rows, cols] tensors.  NaN must sit at the same places on both
    sides (a NaN reference element is compared only for NaN-ness).
    max_rel: the element-wise bar (error relative to max(|o|, rms(o))).
    mae: mean-absolute-error bar, times rms(o) when mae_rel.
    flip_budget: fraction of elements allowed above max_rel (each <= flip_max).
    cols: apply the MAE bar and the flip budget to every column as well.
    groups: optional int tensor [rows] of row-group ids; the MAE bar and the
      flip budget then also hold inside every group.
    """
    g, o = got.double().cpu(), ref.double().cpu()
    if g.dim() == 1:
        g, o = g.view(-1, 1), o.view(-1, 1)
    out = []
    if g.shape != o.shape:
        return [f"{what}: shape {tuple(g.shape)} != {tuple(o.shape)}"]
    nan_o, nan_g = torch.isnan(o), torch.isnan(g)
    if not torch.equal(nan_o, nan_g):
        out.append(f"{what}: NaN at {int((nan_o != nan_g).sum())} places where the other side has none")
    inf_o = torch.isinf(o)
    if not torch.equal(g[inf_o], o[inf_o]):
        out.append(f"{what}: infinities differ")
    fin = torch.isfinite(o)
    if not bool(torch.isfinite(g[fin]).all()):
        out.append(f"{what}: non-finite values where the reference is finite")
        return out
    if not bool(fin.any()):
        return out
    rms = _rms(o[fin])
    bar_mae = mae * (rms.item() if mae_rel else 1.0)
    diff = torch.where(fin, (g - o).abs(), torch.zeros_like(g))
    rel = diff / torch.maximum(o.abs(), rms)
    rel = torch.where(fin, rel, torch.zeros_like(rel))
    flips = rel > max_rel
    n = int(fin.sum())
    nflip = int(flips.sum())
    allowed = int(flip_budget * n)
    if nflip > allowed:
        out.append(f"{what}: {nflip} of {n} elements above max_rel {max_rel} (budget {allowed}); "
                   f"max_rel {rel.max().item():.3e}")
    if nflip and rel.max().item() > flip_max:
        out.append(f"{what}: max_rel {rel.max().item():.3e} > {flip_max}")
    m = diff.sum().item() / n
    if m > bar_mae:
        out.append(f"{what}: MAE {m:.3e} > {bar_mae:.3e}")

    # A column's or a row group's MAE may not exceed the larger of the bar and
    # four times the whole tensor's MAE (the contract's bar is on the whole
    # tensor; the local check looks for a column or a tile far worse than the
    # rest), plus room for one element at the element-wise bar (with few rows
    # a single one-ulp flip moves a column's mean).
    local_mae = max(bar_mae, 4 * m)
    if cols and g.shape[0] > 1:
        cnt = fin.sum(dim=0).clamp_min(1).double()
        col_mae = diff.sum(dim=0) / cnt
        col_flip = flips.sum(dim=0).double()
        lim = torch.clamp(flip_budget * 8 * cnt, min=2.0 if flip_budget > 0 else 0.0)
        col_big = torch.where(fin, o.abs(), torch.zeros_like(o)).amax(dim=0)
        col_lim = local_mae + max_rel * torch.maximum(col_big, rms) / cnt
        worst = int((col_mae / col_lim).argmax())
        if col_mae[worst].item() > col_lim[worst].item():
            out.append(f"{what}: column {worst} MAE {col_mae[worst].item():.3e} > {col_lim[worst].item():.3e}")
        badc = (col_flip > lim).nonzero().flatten()
        if badc.numel():
            c = int(badc[0])
            out.append(f"{what}: column {c} has {int(col_flip[c])} of {int(cnt[c])} elements above max_rel")
    if groups is not None:
        # A row group (a kernel tile) is judged by the median over its rows of
        # the row's MAE and of the row's share of elements above max_rel: a
        # wrong tile moves all of its rows, while in the w4a8 path a single
        # row can legitimately move as a whole (one e4m3 step of a large H
        # element reaches every column of that row's Y).
        gid = torch.as_tensor(groups).view(-1).long().cpu()
        rcnt = fin.sum(dim=1).clamp_min(1).double()
        row_mae = diff.sum(dim=1) / rcnt
        row_flip = flips.sum(dim=1).double() / rcnt
        row_big = torch.where(fin, o.abs(), torch.zeros_like(o)).amax(dim=1)
        for gv in torch.unique(gid).tolist():
            rows = (gid == gv).nonzero().flatten()
            if int(fin[rows].sum()) == 0:
                continue
            gm = row_mae[rows].median().item()
            gf = row_flip[rows].median().item()
            big = row_big[rows].max().item()
            ncol = rcnt[rows].max().item()
            glim = local_mae + max_rel * max(big, rms.item()) / ncol
            if gm > glim:
                out.append(f"{what}: row group {gv} median row MAE {gm:.3e} > {glim:.3e}")
                break
            if gf > flip_budget * 8:
                out.append(f"{what}: row group {gv}: median row has {gf:.2e} of its elements above max_rel")
                break
    return out


def assert_elementwise(got, ref, what="y", **kw):
    m = metrics(got, ref)
    log(f"  {what}: max_rel={m['max_rel']:.3e} mae={m['mae']:.3e} rms={m['rms']:.3e} "
        f"inf_ratio={m['inf_ratio']:.3e}")
    fails = elementwise_failures(got, ref, what=what, **kw)
    assert not fails, "; ".join(fails)
    return m


def assert_parity(got, ref, max_rel=2e-2, mae=1e-3, what="y", groups=None):
    """The bf16 bar on a layer output (every element, every column, every row group)."""
    return assert_elementwise(got, ref, what=what, max_rel=max_rel, mae=mae, groups=groups)


def assert_intermediate(got, ref, what, groups=None, max_rel=2e-2):
    """The bf16 bar on an intermediate (MAE relative to the tensor's RMS)."""
    return assert_elementwise(got, ref, what=what, max_rel=max_rel, mae=1e-3, mae_rel=True, groups=groups)


# w4a8 budgets.  Outputs: on the oracle alone (ascending vs descending K) no
# element exceeds 5e-2; 1e-3 of the elements may.  Codes of z: a one-ulp bf16
# difference of z moves its code only across an e4m3 rounding boundary (about
# 1 in 32 such differences; 3e-5 of the codes at the prefill shape): 1e-3.
# Codes of H: such a flipped z code shifts every H element of that token and
# expert by ~1e-3 absolute, which moves the codes of H elements that sit near
# a rounding boundary or far below their block's maximum; measured on the MI355X
# at 2.2e-3 of H's codes at the prefill shape: 1e-2.
W4A8_FLIP_BUDGET = 1e-3
W4A8_CODE_BUDGET = 1e-3
W4A8_H_CODE_BUDGET = 1e-2
# Size of a single w4a8 element's excursion: the OCP scale rule puts a
# block's largest value at 256..512 times the scale while e4m3 stops at 448,
# so a one-ulp bf16 difference at a block maximum can decide a 1/8 clip of it,
# and an H element feeds every column of its row's Y; between two valid
# orders of the oracle a Y element moved by 0.14, on the MI355X by 0.19.  The
# cap still rejects a zeroed (1.0) or sign-flipped (2.0) element.
W4A8_FLIP_MAX = 0.5


def assert_w4a8(got, ref, what="y", groups=None, mae_rel=False):
    """The MXFP4 w4a8 bar: element-wise 5e-2 with the flip budget above."""
    return assert_elementwise(got, ref, what=what, max_rel=5e-2, mae=1e-3, mae_rel=mae_rel,
                              flip_budget=W4A8_FLIP_BUDGET, flip_max=W4A8_FLIP_MAX, groups=groups)


def mxfp8_values(codes, scales):
    """Dequantised MXFP8 values (float64) of e4m3fn codes [rows, K] and e8m0
    scales [rows, K/32] (scale 255 -> NaN)."""
    codes, scales = codes.cpu(), scales.cpu()
    el = codes.contiguous().view(torch.float8_e4m3fn).to(torch.float64)
    sc = torch.pow(2.0, scales.to(torch.float64) - 127)
    sc = torch.where(scales == 255, torch.full_like(sc, float("nan")), sc)
    return el * sc.repeat_interleave(32, dim=-1)


def mxfp8_failures(codes, scales, rcodes, rscales, budget=W4A8_CODE_BUDGET, what="zq"):
    """MXFP8 encodings compared through their values [rows, K]: NaN blocks at
    the same places; at most ``budget`` of the values differ, overall and
    (times 8) in every column; each difference is at most one e4m3 ulp at the
    larger of the two values, or one e4m3 ulp of the block's largest value /
    8 for values far below it (the format's precision is relative to its
    block); block scales differ by at most one binade."""
    a, b = mxfp8_values(codes, scales), mxfp8_values(rcodes, rscales)
    out = []
    na, nb = torch.isnan(a), torch.isnan(b)
    if not torch.equal(na, nb):
        out.append(f"{what}: NaN blocks differ at {int((na != nb).sum())} elements")
    fin = ~(na | nb)
    sc = torch.maximum(scales.cpu().to(torch.int64), rscales.cpu().to(torch.int64)).repeat_interleave(32, dim=-1)
    X = torch.pow(2.0, (sc - 127).to(torch.float64))

    def e4m3_ulp(mag):                                       # mag in units of the block scale
        return torch.pow(2.0, torch.floor(torch.log2(mag.clamp_min(2.0 ** -6))) - 3)

    big = torch.maximum(a.abs(), b.abs())
    blk = torch.where(fin, big, torch.zeros_like(big)).view(*big.shape[:-1], -1, 32).amax(dim=-1)
    blk = blk.repeat_interleave(32, dim=-1)
    tol = torch.maximum(e4m3_ulp(big / X), e4m3_ulp(blk / X) / 8) * X
    d = (a - b).abs()
    diff = fin & (a != b)
    n = int(fin.sum())
    if int(diff.sum()) > int(budget * n):
        out.append(f"{what}: {int(diff.sum())} of {n} values differ (budget {int(budget * n)})")
    if diff.dim() == 2 and diff.shape[0] > 1:
        per_col = diff.sum(dim=0).double()
        lim = torch.clamp(8 * budget * fin.sum(dim=0).double(), min=2.0)
        badc = (per_col > lim).nonzero().flatten()
        if badc.numel():
            c = int(badc[0])
            out.append(f"{what}: column {c} has {int(per_col[c])} differing values")
    over = diff & (d > tol * (1 + 1e-12))
    if bool(over.any()):
        out.append(f"{what}: {int(over.sum())} values differ by more than their tolerance")
    sdiff = (scales.cpu().to(torch.int64) - rscales.cpu().to(torch.int64)).abs()
    if int(sdiff.max()) > 1 if sdiff.numel() else False:
        out.append(f"{what}: a block scale differs by {int(sdiff.max())} binades")
    return out


def assert_mxfp8(codes, scales, rcodes, rscales, what="zq", budget=W4A8_CODE_BUDGET):
    fails = mxfp8_failures(codes, scales, rcodes, rscales, budget=budget, what=what)
    a, b = mxfp8_values(codes, scales), mxfp8_values(rcodes, rscales)
    nd = int(((a != b) & ~(torch.isnan(a) | torch.isnan(b))).sum())
    log(f"  {what}: {nd} of {a.numel()} MXFP8 values differ")
    assert not fails, "; ".join(fails)


def assert_w4a8_codes(zq, zs, rzq, rzs, hq, hsc, rhq, rhqs, row_tok, exact_z=False):
    """The MXFP8 codes of a w4a8 forward against the oracle's.  zq/zs: FC1's
    input codes and scales by token; hq/hsc: FC2's input by routed row, with
    row_tok[i] the index (into the token rows) of routed row i's token.
    z's codes within their budget (exact_z: bit for bit, when the quantiser
    reads the given activations); H's codes are compared on the rows whose
    token has an identical MXFP8 z row on both sides: a token whose z codes
    differ (a one-ulp bf16 difference of z crossing an e4m3 rounding
    boundary) feeds FC1 a different input, which shifts all its H values, and
    is judged through the layer's outputs instead (rhat, y).  Returns the mask
    of the routed rows whose token's z codes are identical."""
    if exact_z:
        assert torch.equal(zq, rzq) and torch.equal(zs, rzs), "MXFP8 codes of the given rows differ"
    else:
        assert_mxfp8(zq, zs, rzq, rzs, what="zq")
    same = (zq == rzq).all(dim=1) & (zs == rzs).all(dim=1)
    rows_same = same[torch.as_tensor(row_tok).long()]
    log(f"  {int((~same).sum())} of {same.numel()} tokens have an MXFP8 z row that differs")
    assert_mxfp8(hq[rows_same], hsc[rows_same], rhq[rows_same], rhqs[rows_same], what="hq",
                 budget=W4A8_H_CODE_BUDGET)
    return rows_same


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


def covering_tokens(offsets, sorted_row, k, T, dense_tile=256, expert_tile=192, spread=97):
    """Tokens whose evaluation touches every tile of the layer's GEMMs: the
    first and last token of every ``dense_tile``-row tile of the dense
    projections, and, for every expert, the token of the first row of each of
    its ``expert_tile``-row tiles and of its last row (rows in permuted
    order); plus every ``spread``-th token."""
    off = torch.as_tensor(offsets).long().cpu()
    srow = torch.as_tensor(sorted_row).long().cpu()
    pick = set(range(0, T, spread))
    for m in range(0, T, dense_tile):
        pick |= {m, min(T - 1, m + dense_tile - 1)}
    E = off.numel() - 1
    for e in range(E):
        a, b = int(off[e]), int(off[e + 1])
        if b <= a:
            continue
        for p in list(range(a, b, expert_tile)) + [b - 1]:
            pick.add(int(srow[p]) // k)
    return sorted(pick)


def slot_positions(tokens, row_pos, k):
    """Permuted-row indices of the slots of ``tokens``: entry i*k + j is the
    position of row tokens[i]*k + j (the oracle's sampled H/Y row order)."""
    rp = torch.as_tensor(row_pos).long().cpu()
    t = torch.as_tensor(tokens, dtype=torch.int64).view(-1, 1)
    return rp[(t * k + torch.arange(k).view(1, -1)).view(-1)]


def expert_tile_ids(positions, offsets, expert_tile=192):
    """Group id (expert tile) of permuted rows ``positions``."""
    off = torch.as_tensor(offsets).long().cpu()
    p = torch.as_tensor(positions).long().cpu()
    e = torch.searchsorted(off, p, right=True) - 1
    return e * 100000 + (p - off[e]) // expert_tile
