"""GPU parity at the full sizes the bench times.

Routing is compared bit for bit over the whole batch.  The layer's
intermediates and outputs are compared element by element on tokens chosen so
that every tile of every GEMM is touched: the first and last token of every
256-row tile of the dense projections, and the tokens of the first row of
every 192-row tile of every expert and of each expert's last row (plus a
spread); one expert-parallel rank's share is compared on every row.  A last
case puts the activations and the expert outputs past 4 GiB, where element
offsets no longer fit 32 bits.
"""
import pytest
import torch

import oracle
import workloads as W
from tests.gpu_helpers import check_layer, check_routing, run_gpu_layer
from tests.parity import assert_parity, covering_tokens, log, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import latentmoe_expert_layer_amd  # noqa: F401  (fails loudly if the library is not built)
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    yield


@pytest.mark.parametrize("name", ["prefill", "prefill_bf16_16k", "prefill_mxfp4", "prefill_w4a16"])
def test_full_size_every_tile(name):
    cfg = W.CONFIGS[name]
    log(f"full-size {name}: {cfg}")
    inp_dev = W.make_inputs(cfg, device="cuda")
    r, y, views = run_gpu_layer(inp_dev)
    ids, w = check_routing(r, inp_dev["logits"], cfg.k, cfg.E)
    inp = to_host(inp_dev)
    del inp_dev
    off, srow, _ = oracle.permute(ids, cfg.E)
    toks = covering_tokens(off, srow, cfg.k, cfg.T)
    log(f"  {len(toks)} tokens cover every dense and expert tile")
    check_layer(inp, ids, w, y, views, tokens=toks)


def test_ep_share_every_row():
    """One expert-parallel rank's share (56 experts, 16,384 Zipf-loaded rows):
    every row of Y and of the weighted output."""
    cfg = W.CONFIGS["ep_share"]
    log(f"ep_share rows mode: {cfg}")
    inp_dev = W.make_inputs(cfg, device="cuda")
    r, y, views = run_gpu_layer(inp_dev)
    inp = to_host(inp_dev)
    check_routing(r, inp["ids"].view(-1), 1, cfg.E, weights=inp["weights"])
    check_layer(inp, inp["ids"], inp["weights"], y, views)


def test_rows_mode_past_4_gib():
    """1.1 M received rows at latent 2048: x, Y and the output each span
    4.5 GB (2.25 G elements), so row offsets past 2^31 elements and 2^32 bytes
    are exercised.  Checked: the permutation of all rows by the properties of
    a stable counting sort, and Y and the output on the rows at both ends of
    the buffers and at every expert's first and last permuted row."""
    R, E, l, I = 1_100_000, 56, 2048, 512
    cfg = W.custom("rows_4gib", T=R, d=0, l=l, E=E, k=1, S=0, I=I, Is=0, rows_mode=True, norm=False,
                   zipf_s=1.1, seed=3)
    assert R * l * 2 > 2 ** 32
    log(f"rows mode past 4 GiB: {cfg}")
    inp_dev = W.make_inputs(cfg, device="cuda")
    r, y, views = run_gpu_layer(inp_dev)
    ids = inp_dev["ids"].view(-1).cpu().long()
    off = torch.zeros(E + 1, dtype=torch.int64)
    off[1:] = torch.bincount(ids, minlength=E).cumsum(0)
    assert torch.equal(r.offsets.cpu().long(), off)
    srt = torch.sort(ids, stable=True).indices
    assert torch.equal(r.sorted_row.cpu().long(), srt)
    rp = torch.empty_like(srt)
    rp[srt] = torch.arange(R)
    assert torch.equal(r.row_pos.cpu().long(), rp)
    # rows to check: both ends of the received order and of the permuted order,
    # and each expert's first and last permuted rows
    pick = {0, 1, R // 2, R - 2, R - 1}
    for p in list(range(R - 6, R)) + list(range(0, 6)):
        pick.add(int(srt[p]))
    for e in range(E):
        if off[e + 1] > off[e]:
            pick |= {int(srt[off[e]]), int(srt[off[e + 1] - 1])}
    pick = sorted(pick)
    log(f"  checking {len(pick)} rows; largest output row offset {max(pick) * l * 2 / 2**30:.2f} GiB, "
        f"largest Y row offset {int(rp[pick].max()) * l * 2 / 2**30:.2f} GiB")
    # the oracle evaluates just these rows (inputs drawn by the generator,
    # rows selected; the expert weights whole)
    sub = {"cfg": W.custom("rows_4gib_pick", T=len(pick), d=0, l=l, E=E, k=1, S=0, I=I, Is=0,
                           rows_mode=True, norm=False),
           "x": inp_dev["x"][pick].cpu(), "ids": inp_dev["ids"][pick].cpu(),
           "weights": inp_dev["weights"][pick].cpu()}
    for n in ("w1", "w3", "w2"):
        sub[n] = inp_dev[n].cpu()
    ref = oracle.layer(sub, sub["ids"], sub["weights"], intermediates=True,
                       row_pos=torch.arange(len(pick), dtype=torch.int32))
    assert_parity(y[pick].cpu(), ref["y"], what="y (rows past 4 GiB)")
    assert_parity(views["Y"][rp[pick]].cpu(), ref["Y"], what="Y (rows past 4 GiB)")
