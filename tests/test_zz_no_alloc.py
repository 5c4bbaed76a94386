"""latent_moe_layer_noalloc (the entry point that allocates nothing: its
workspaces live in the library's static device scratch) against
latent_moe_layer (caller workspaces), through the C ABI: routing outputs and
the layer output bit for bit, on two calls in a row, the second with a
smaller batch; then the call captured in a HIP graph, every replay equal to
the eager result."""
import pytest
import torch

import workloads as W
from tests.parity import log, poison_

pytestmark = pytest.mark.gpu

CASES = [
    # the decode batch, then a smaller ragged one (fewer tokens and experts, other widths)
    W.CONFIGS["decode"],
    W.custom("noalloc_small", T=77, d=128, l=320, E=40, k=8, S=2, I=192, Is=64),
]


@pytest.fixture(scope="module")
def lm():
    import latentmoe_expert_layer_amd as m
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return m


def outputs(cfg):
    T, E, k = cfg.T, cfg.E, cfg.k
    return dict(ids=poison_(torch.empty(T, k, dtype=torch.int32, device="cuda")),
                w=poison_(torch.empty(T, k, dtype=torch.float32, device="cuda")),
                srow=poison_(torch.empty(T * k, dtype=torch.int32, device="cuda")),
                rpos=poison_(torch.empty(T * k, dtype=torch.int32, device="cuda")),
                off=poison_(torch.empty(E + 1, dtype=torch.int32, device="cuda")),
                y=poison_(torch.empty(T, cfg.d, dtype=torch.bfloat16, device="cuda")))


def call_args(lm, cfg, inp, out):
    P = lambda t: None if t is None else t.data_ptr()
    ra = lm.RouteArgs(T=cfg.T, E=cfg.E, k=cfg.k, logits=P(inp["logits"]), topk_ids=P(out["ids"]),
                      topk_w=P(out["w"]), sorted_row=P(out["srow"]), row_pos=P(out["rpos"]), offsets=P(out["off"]))
    fa = lm.ForwardArgs(d=cfg.d, l=cfg.l, I=cfg.I, S=cfg.S, Is=cfg.Is, wfmt=lm.LMOE_WFMT_BF16, norm_eps=cfg.eps,
                        x=P(inp["x"]), w_in=P(inp["w_in"]), w1=P(inp["w1"]), w3=P(inp["w3"]), w2=P(inp["w2"]),
                        norm_w=P(inp.get("norm_w")), w_out=P(inp["w_out"]), ws1=P(inp.get("ws1")),
                        ws3=P(inp.get("ws3")), ws2=P(inp.get("ws2")), y=P(out["y"]))
    return ra, fa


def reference(lm, cfg, inp):
    r, y = lm.layer(inp["x"], None, cfg.k, inp["w1"], inp["w3"], inp["w2"], w_in=inp["w_in"], w_out=inp["w_out"],
                    ws1=inp.get("ws1"), ws3=inp.get("ws3"), ws2=inp.get("ws2"), norm_w=inp.get("norm_w"),
                    eps=cfg.eps, logits=inp["logits"])
    torch.cuda.synchronize()
    return dict(ids=r.topk_ids, w=r.topk_w, srow=r.sorted_row, rpos=r.row_pos, off=r.offsets, y=y)


def assert_same(got, ref, what):
    for n in ("ids", "w", "srow", "rpos", "off", "y"):
        a, b = got[n], ref[n]
        if a.dtype == torch.bfloat16:
            a, b = a.view(torch.int16), b.view(torch.int16)
        assert torch.equal(a, b), f"{what}: {n} differs from latent_moe_layer"


def test_noalloc_equals_layer_on_two_calls_in_a_row(lm):
    stream = torch.cuda.current_stream().cuda_stream
    for i, cfg in enumerate(CASES):
        log(f"call {i}: {cfg}")
        inp = W.make_inputs(cfg, device="cuda")
        ref = reference(lm, cfg, inp)
        out = outputs(cfg)
        ra, fa = call_args(lm, cfg, inp, out)
        lm.latent_moe_layer_noalloc(ra, None, None, fa, stream)
        torch.cuda.synchronize()
        assert_same(out, ref, f"call {i}")


def test_noalloc_graph_replay(lm):
    """Captured in a HIP graph: every replay, with eager work and
    synchronisations in between, equals the eager result."""
    cfg = CASES[1]
    inp = W.make_inputs(cfg, device="cuda")
    ref = reference(lm, cfg, inp)
    out = outputs(cfg)
    ra, fa = call_args(lm, cfg, inp, out)
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    with torch.cuda.graph(g, stream=cap):
        lm.latent_moe_layer_noalloc(ra, None, None, fa, torch.cuda.current_stream().cuda_stream)
    for rep in range(3):
        for t in out.values():
            poison_(t)
        junk = torch.randn(1 << 20, device="cuda").sum()   # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert_same(out, ref, f"replay {rep}")
        del junk


def test_noalloc_refuses_a_batch_beyond_its_scratch(lm):
    cfg = W.custom("noalloc_big", T=4096, d=512, l=256, E=896, k=16, S=2, I=256, Is=256)
    inp = W.make_inputs(cfg, device="cuda")
    out = outputs(cfg)
    before = out["y"].clone()
    ra, fa = call_args(lm, cfg, inp, out)
    with pytest.raises(lm.LatentMoeError) as ei:
        lm.latent_moe_layer_noalloc(ra, None, None, fa, torch.cuda.current_stream().cuda_stream)
    assert ei.value.code == lm.LMOE_EUNSUPPORTED
    torch.cuda.synchronize()
    assert torch.equal(out["y"].view(torch.int16), before.view(torch.int16))
