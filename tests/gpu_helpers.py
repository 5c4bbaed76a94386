"""Shared machinery of the GPU parity tests: run the layer through the C ABI on
poisoned buffers, read the intermediates the forward left in its workspace
(through latent_moe_forward_workspace_layout), and compare each of them with
the oracle's, element by element, grouped by the tiles the kernels work on.
"""
import torch

import oracle
from tests.parity import (assert_intermediate, assert_parity, assert_w4a8, assert_w4a8_codes, expert_tile_ids, log,
                          poison_, slot_positions)

SKINNY_BM, TILED_BM, SMALL_M = 16, 192, 512


def lm():
    import latentmoe_expert_layer_amd as m  # fails loudly if the library is not built
    return m


def wfmt_of(cfg):
    m = lm()
    if not cfg.mxfp4:
        return m.LMOE_WFMT_BF16
    return m.LMOE_WFMT_MXFP4_W4A16 if cfg.w4a16 else m.LMOE_WFMT_MXFP4


def expert_tile_rows(cfg):
    """Row cut of the grouped kernels' tiles for this configuration."""
    R = cfg.T * cfg.k
    if cfg.mxfp4 and not cfg.w4a16:
        return TILED_BM
    if R <= 32 * cfg.E:
        return SKINNY_BM
    return TILED_BM


def dense_tile_rows(cfg):
    return SKINNY_BM if cfg.T <= SMALL_M else 256


def gpu_route(logits=None, k=1, **kw):
    m = lm()
    T = logits.shape[0] if logits is not None else kw["ids"].shape[0]
    E = logits.shape[1] if logits is not None else kw["E"]
    ws = poison_(torch.empty(m.route_workspace_size(T, E, k), dtype=torch.uint8, device="cuda"))
    r = m.route(logits, k, workspace=ws, **kw)
    torch.cuda.synchronize()
    return r


def run_gpu_layer(inp_dev, norm=True):
    """route + forward on poisoned output and workspace buffers; returns
    (routing, y, views of the workspace intermediates)."""
    m = lm()
    cfg = inp_dev["cfg"]
    T = cfg.T
    mx = cfg.mxfp4
    wfmt = wfmt_of(cfg)
    w1, w3, w2 = (inp_dev[n + ("q" if mx else "")] for n in ("w1", "w3", "w2"))
    wts = dict(s1=inp_dev.get("s1"), s3=inp_dev.get("s3"), s2=inp_dev.get("s2"), mxfp4=mx, w4a16=cfg.w4a16,
               I=cfg.I)
    if cfg.rows_mode:
        r = gpu_route(None, 1, ids=inp_dev["ids"], weights=inp_dev["weights"], E=cfg.E)
        nbytes = m.forward_workspace_size(T, cfg.E, 1, 0, cfg.l, cfg.I, 0, 0, wfmt, True)
        ws = poison_(torch.empty(max(nbytes, 256), dtype=torch.uint8, device="cuda"))
        y = poison_(torch.empty(T, cfg.l, dtype=torch.bfloat16, device="cuda"))
        m.forward(r, inp_dev["x"], w1, w3, w2, y=y, workspace=ws, **wts)
        torch.cuda.synchronize()
        views = m.workspace_views(ws, T, cfg.E, 1, 0, cfg.l, cfg.I, 0, 0, wfmt, True)
        return r, y, views
    r = gpu_route(inp_dev["logits"], cfg.k)
    nbytes = m.forward_workspace_size(T, cfg.E, cfg.k, cfg.d, cfg.l, cfg.I, cfg.S, cfg.Is, wfmt, False)
    ws = poison_(torch.empty(max(nbytes, 256), dtype=torch.uint8, device="cuda"))
    y = poison_(torch.empty(T, cfg.d, dtype=torch.bfloat16, device="cuda"))
    m.forward(r, inp_dev["x"], w1, w3, w2, w_in=inp_dev["w_in"], w_out=inp_dev["w_out"],
              ws1=inp_dev.get("ws1"), ws3=inp_dev.get("ws3"), ws2=inp_dev.get("ws2"),
              norm_w=inp_dev.get("norm_w") if norm else None, eps=cfg.eps, y=y, workspace=ws, **wts)
    torch.cuda.synchronize()
    views = m.workspace_views(ws, T, cfg.E, cfg.k, cfg.d, cfg.l, cfg.I, cfg.S, cfg.Is, wfmt, False)
    return r, y, views


def check_routing(r, logits_or_ids, k, E, weights=None):
    if weights is None:
        ids_ref, w_ref = oracle.route(logits_or_ids.cpu(), k)
        assert torch.equal(r.topk_ids.cpu(), ids_ref), "router ids differ"
        dw = (r.topk_w.cpu().double() - w_ref.double()).abs().max().item()
        assert dw <= 2e-6, f"combine weights differ by {dw}"
    else:
        ids_ref, w_ref = logits_or_ids.cpu(), weights.cpu()
    off, srow, rpos = oracle.permute(ids_ref, E)
    assert torch.equal(r.offsets.cpu(), off), "offsets differ"
    assert torch.equal(r.sorted_row.cpu(), srow), "sorted_row differs"
    assert torch.equal(r.row_pos.cpu(), rpos), "row_pos differs"
    return ids_ref, w_ref


def check_layer(inp_host, ids, w, y, views, tokens=None, act_quant=None, norm=True):
    """Compares y and every intermediate in ``views`` with the oracle's, for
    all tokens or for ``tokens``.  The routing (ids, w) is the oracle's (the
    tests check beforehand that the GPU's equals it bit for bit)."""
    cfg = inp_host["cfg"]
    w4a8 = cfg.mxfp4 and not cfg.w4a16
    aq = w4a8 if act_quant is None else act_quant
    k = cfg.k
    offsets, _, row_pos = oracle.permute(ids, cfg.E)
    inp = inp_host if norm else {kk: v for kk, v in inp_host.items() if kk != "norm_w"}
    if tokens is None:
        ref = oracle.layer(inp, ids, w, row_pos=row_pos, intermediates=True, act_quant=aq)
        tok = torch.arange(cfg.T)
        pos = torch.arange(cfg.T * k)
        # the compared H/Y rows are in permuted order: row p is token sorted_row[p] // k
        row_tok = oracle.permute(ids, cfg.E)[1].long() // k
    else:
        ref = oracle.layer(inp, ids, w, eval_tokens=tokens, intermediates=True, act_quant=aq)
        tok = torch.as_tensor(tokens, dtype=torch.int64)
        pos = slot_positions(tokens, row_pos, k)
        # row i*k + j is slot j of tokens[i]
        row_tok = torch.arange(tok.numel()).repeat_interleave(k)
    rgroups = expert_tile_ids(pos, offsets, expert_tile_rows(cfg))
    # rows mode (k = 1): a row's output belongs to its expert's tile
    tgroups = rgroups if cfg.rows_mode else tok // dense_tile_rows(cfg)
    g = {n: v.cpu() for n, v in views.items()}
    log(f"  comparing {tok.numel()} tokens, {pos.numel()} routed rows")
    if "z" in g:
        assert_intermediate(g["z"][tok], ref["z"], "z", groups=tgroups)
    if "hs" in g and g["hs"].numel():
        assert_intermediate(g["hs"][tok], ref["hs"], "hs", groups=tgroups)
    if "H" in g:
        assert_intermediate(g["H"][pos], ref["H"], "H", groups=rgroups)
    if w4a8:
        same = assert_w4a8_codes(g["zq"][tok], g["zs"][tok], ref["zq"], ref["zqs"], g["hq"][pos], g["hsc"][pos],
                                 ref["hq"], ref["hqs"], row_tok, exact_z=cfg.rows_mode)
        # Y on the rows whose FC1 input codes are identical on both sides
        assert_w4a8(g["Y"][pos][same], ref["Y"][same], what="Y", groups=rgroups[same], mae_rel=True)
        if "rhat" in g:
            assert_w4a8(g["rhat"][tok], ref["rhat"], what="rhat", groups=tgroups, mae_rel=True)
        yg = y.cpu()[tok] if y.shape[0] == cfg.T else y.cpu()
        assert_w4a8(yg, ref["y"], what="y", groups=tgroups)
    else:
        assert_intermediate(g["Y"][pos], ref["Y"], "Y", groups=rgroups)
        if "rhat" in g:
            assert_intermediate(g["rhat"][tok], ref["rhat"], "rhat", groups=tgroups)
        yg = y.cpu()[tok] if y.shape[0] == cfg.T else y.cpu()
        assert_parity(yg, ref["y"], groups=tgroups)
    return ref
