"""C ABI checks that need no GPU: the library loads, exports every entry point
the header declares, sizes workspaces, and rejects invalid arguments before
any launch (no compute call is made here)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "latent_moe.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(latent_moe_\w+)\s*\(", text)))


def test_header_declares_the_three_calls():
    names = declared_functions()
    for n in ("latent_moe_route", "latent_moe_forward", "latent_moe_free"):
        assert n in names


def test_library_exports_every_declared_symbol():
    import latentmoe_expert_layer_amd as lm
    lib = ctypes.CDLL(lm.LIB_PATH)
    for n in declared_functions():
        assert hasattr(lib, n), f"{n} not exported"


def test_oracle_is_not_linked_into_the_product():
    import latentmoe_expert_layer_amd as lm
    with open(lm.LIB_PATH, "rb") as f:
        blob = f.read()
    assert b"lmoe_oracle" not in blob


def test_workspace_sizes():
    import latentmoe_expert_layer_amd as lm
    a = lm.route_workspace_size(8192, 896, 16)
    b = lm.route_workspace_size(256, 896, 16)
    assert a > b > 0
    assert lm.route_workspace_size(-1, 896, 16) == 0
    assert lm.route_workspace_size(10, 4, 8) == 0          # k > E
    f = lm.forward_workspace_size(8192, 896, 16, 7168, 2048, 512, 2, 512)
    # z + hs + H + Y + rhat in bf16
    need = 2 * (8192 * 2048 + 8192 * 1024 + 131072 * 512 + 131072 * 2048 + 8192 * 2048)
    assert need <= f <= need + 16 * 256
    r = lm.forward_workspace_size(16384, 56, 1, 0, 2048, 512, 0, 0, rows_mode=True)
    assert 2 * (16384 * 512 + 16384 * 2048) <= r
    # MXFP4 w4a16 keeps bf16 intermediates: the bf16 layout; w4a8 adds MXFP8
    # copies but no bf16 H; unknown formats size to 0
    bf = lm.forward_workspace_size(256, 896, 16, 512, 256, 256, 2, 256, lm.LMOE_WFMT_BF16)
    assert lm.forward_workspace_size(256, 896, 16, 512, 256, 256, 2, 256, lm.LMOE_WFMT_MXFP4_W4A16) == bf
    assert lm.forward_workspace_size(256, 896, 16, 512, 256, 256, 2, 256, lm.LMOE_WFMT_MXFP4) > 0
    assert lm.forward_workspace_size(256, 896, 16, 512, 256, 256, 2, 256, 3) == 0


def _route_args(lm, **kw):
    base = dict(T=4, E=16, k=4, logits=16, ids_in=None, weights_in=None, topk_ids=32, topk_w=48,
                sorted_row=64, row_pos=80, offsets=96, workspace=112, workspace_bytes=1 << 20)
    base.update(kw)
    return lm.RouteArgs(**base)


@pytest.mark.parametrize("kw,code", [
    (dict(k=0), 1), (dict(k=65, E=100), 1), (dict(E=3), 1), (dict(T=-1), 1),
    (dict(logits=None), 1),                               # neither logits nor ids
    (dict(T=0, k=0), 1),                                  # dims are checked even when empty
    (dict(ids_in=128, weights_in=144), 1),                # both logits and ids
    (dict(logits=None, ids_in=128, weights_in=None, k=1), 1),
    (dict(logits=None, ids_in=128, weights_in=144, k=2), 1),
    (dict(topk_ids=None), 1), (dict(sorted_row=None), 1),
    (dict(logits=17), 1),                                 # misaligned
    (dict(workspace_bytes=16), 1),                        # workspace too small
    (dict(E=2000, k=4), 2),                               # logits mode E limit
    (dict(logits=None, ids_in=128, weights_in=144, k=1, E=5000), 2),
])
def test_route_rejects_invalid_arguments(kw, code):
    import latentmoe_expert_layer_amd as lm
    with pytest.raises(lm.LatentMoeError) as ei:
        lm.latent_moe_route(_route_args(lm, **kw))
    assert ei.value.code == code, lm.latent_moe_last_error()
    assert lm.latent_moe_last_error()


def test_route_with_empty_batch_needs_no_launch():
    import latentmoe_expert_layer_amd as lm
    plan = lm.latent_moe_route(_route_args(lm, T=0))
    assert plan
    fa = lm.ForwardArgs(d=512, l=256, I=128, S=1, Is=128, wfmt=0, norm_eps=1e-6, x=16, w_in=32, w1=48,
                        w3=64, w2=80, w_out=96, ws1=112, ws3=128, ws2=144, y=160, workspace=176,
                        workspace_bytes=1 << 20)
    lm.latent_moe_forward(plan, fa)                       # T == 0: OK, nothing enqueued
    lm.latent_moe_forward(plan, lm.ForwardArgs(**{**{f: getattr(fa, f) for f, _ in fa._fields_},
                                                  "x": None, "y": None}))  # pointers unused
    for bad, code in [(dict(l=100), 1), (dict(I=0), 1), (dict(d=65), 1), (dict(S=5), 1),
                      (dict(Is=32), 1), (dict(wfmt=7), 1), (dict(w_out=None), 1), (dict(l=8192), 2)]:
        args = lm.ForwardArgs(**{**{f: getattr(fa, f) for f, _ in fa._fields_}, **bad})
        with pytest.raises(lm.LatentMoeError) as ei:
            lm.latent_moe_forward(plan, args)
        assert ei.value.code == code, (bad, lm.latent_moe_last_error())
    # rows mode needs an ids-mode plan
    args = lm.ForwardArgs(**{**{f: getattr(fa, f) for f, _ in fa._fields_}, "w_in": None, "w_out": None})
    with pytest.raises(lm.LatentMoeError):
        lm.latent_moe_forward(plan, args)
    lm.latent_moe_free(plan)
    lm.latent_moe_free(None)
    empty = lm.latent_moe_route(_route_args(lm, T=0, logits=None, topk_ids=None, topk_w=None,
                                            sorted_row=None, row_pos=None, workspace=None))
    lm.latent_moe_free(empty)


def test_forward_rejects_bad_pointers():
    import latentmoe_expert_layer_amd as lm
    # a plan for a non-empty batch cannot be made without a GPU, so build the
    # pointer checks' inputs on an ids-mode plan whose route call fails first
    with pytest.raises(lm.LatentMoeError):
        lm.latent_moe_route(_route_args(lm, T=4, logits=None, ids_in=128, weights_in=144, k=2))


def _layer_fwd(lm, **kw):
    base = dict(d=512, l=256, I=128, S=1, Is=128, wfmt=0, norm_eps=1e-6, x=16, w_in=32, w1=48, w3=64, w2=80,
                w_out=96, ws1=112, ws3=128, ws2=144, y=160, workspace=176, workspace_bytes=1 << 24)
    base.update(kw)
    return lm.ForwardArgs(**base)


@pytest.mark.parametrize("rkw,fkw,gate,logits,code", [
    (dict(), dict(), 192, 208, 1),                              # route logits given: the layer computes them
    (dict(logits=None, ids_in=128, weights_in=144, k=1), dict(), 192, 208, 1),
    (dict(logits=None, topk_ids=None), dict(), 192, 208, 1),
    (dict(logits=None), dict(w_in=None, w_out=None), 192, 208, 1),   # no rows mode
    (dict(logits=None), dict(), None, 208, 1),                  # no gate and no logits
    (dict(), dict(), None, 208, 1),                             # logits given: no logits output
    (dict(logits=None), dict(), None, None, 1),                 # neither gate, logits nor ids
    (dict(), dict(w_in=None, w_out=None), None, None, 1),       # given logits, still no rows mode
    (dict(E=2000), dict(), None, None, 2),                      # given logits: the router's E limit
    (dict(logits=None), dict(), 192, None, 1),                  # no logits buffer
    (dict(logits=None), dict(), 200, 208, 1),                   # misaligned gate
    (dict(logits=None), dict(l=100), 192, 208, 1),
    (dict(logits=None), dict(workspace_bytes=64), 192, 208, 1),
    (dict(logits=None, workspace_bytes=16), dict(), 192, 208, 1),
    (dict(logits=None, E=2000), dict(), 192, 208, 2),           # the router's E limit
])
def test_layer_rejects_invalid_arguments(rkw, fkw, gate, logits, code):
    import latentmoe_expert_layer_amd as lm
    with pytest.raises(lm.LatentMoeError) as ei:
        lm.latent_moe_layer(_route_args(lm, **rkw), gate, logits, _layer_fwd(lm, **fkw))
    assert ei.value.code == code, lm.latent_moe_last_error()


def test_layer_with_empty_batch_returns_and_reuses_a_plan():
    import latentmoe_expert_layer_amd as lm
    ra = _route_args(lm, T=0, logits=None)
    plan = lm.latent_moe_layer(ra, None, None, _layer_fwd(lm))
    assert plan
    assert lm.latent_moe_layer(ra, None, None, _layer_fwd(lm), plan=plan) == plan
    with pytest.raises(lm.LatentMoeError):                      # dims are checked even when empty
        lm.latent_moe_layer(ra, None, None, _layer_fwd(lm, l=100), plan=plan)
    lm.latent_moe_free(plan)


def test_layer_binding_takes_exactly_one_of_gate_and_logits():
    """lm.layer: the router gate and given logits exclude each other (checked
    before any device work)."""
    import torch
    import latentmoe_expert_layer_amd as lm
    x = torch.zeros(4, 64, dtype=torch.bfloat16)
    w = torch.zeros(8, 32, 64, dtype=torch.bfloat16)
    for w_r, logits in ((None, None), (torch.zeros(8, 64, dtype=torch.bfloat16), torch.zeros(4, 8))):
        with pytest.raises(ValueError):
            lm.layer(x, w_r, 2, w, w, w, w_in=torch.zeros(64, 64, dtype=torch.bfloat16),
                     w_out=torch.zeros(64, 64, dtype=torch.bfloat16), logits=logits)


@pytest.mark.parametrize("dims,wfmt,rows", [
    ((8192, 896, 16, 7168, 2048, 512, 2, 512), 0, False),
    ((16384, 896, 16, 7168, 2048, 512, 2, 512), 1, False),
    ((256, 896, 16, 512, 256, 256, 2, 256), 2, False),
    ((256, 896, 16, 512, 384, 256, 2, 256), 2, False),
    ((16384, 56, 1, 0, 2048, 512, 0, 0), 0, True),
    ((16384, 56, 1, 0, 2048, 512, 0, 0), 1, True),
    ((77, 40, 8, 128, 320, 192, 2, 64), 0, False),
])
def test_forward_workspace_layout(dims, wfmt, rows):
    """The intermediates' regions lie inside the workspace, do not overlap,
    and the written bits name what each format writes."""
    import latentmoe_expert_layer_amd as lm
    T, E, k, d, l, I, S, Is = dims
    L = lm.latent_moe_forward_workspace_layout(T, E, k, d, l, I, S, Is, wfmt, rows)
    assert L.total == lm.forward_workspace_size(T, E, k, d, l, I, S, Is, wfmt, rows)
    R = T * k
    sizes = {"z": T * l * 2, "hs": T * S * Is * 2, "H": R * I * 2, "Y": R * l * 2, "rhat": T * l * 2,
             "zq": T * l, "zs": T * l // 32, "hq": R * I, "hsc": R * I // 32}
    bit = {"zs": "zq", "hsc": "hq"}
    spans = []
    for n, nb in sizes.items():
        if L.written & lm.LMOE_WS_BITS[bit.get(n, n)]:
            off = getattr(L, n)
            assert off % 256 == 0 and off + nb <= L.total, n
            spans.append((off, off + nb, n))
    spans.sort()
    for (a0, a1, na), (b0, b1, nb_) in zip(spans, spans[1:]):
        assert a1 <= b0, (na, nb_)
    w = L.written
    assert bool(w & lm.LMOE_WS_BITS["Y"])
    assert bool(w & lm.LMOE_WS_BITS["z"]) == (not rows)
    assert bool(w & lm.LMOE_WS_BITS["zq"]) == (wfmt == 1)
    assert bool(w & lm.LMOE_WS_BITS["H"]) == (wfmt == 0 or (wfmt == 2 and not (l == 256 and I == 256)))
    with pytest.raises(lm.LatentMoeError):
        lm.latent_moe_forward_workspace_layout(T, E, 0, d, l, I, S, Is, wfmt, rows)


def test_noalloc_rejects_workspaces_and_oversized_batches():
    """latent_moe_layer_noalloc refuses caller workspaces (EINVAL) and batches
    whose workspaces exceed its static scratch (EUNSUPPORTED) before any HIP
    call, so this runs without a GPU; the pointers are never dereferenced."""
    import latentmoe_expert_layer_amd as lm
    fake = 1 << 20   # 16-byte aligned stand-in addresses, never read
    T, E, k, d, l, I, S, Is = 256, 896, 16, 512, 256, 256, 2, 256

    def args(T, ws=None):
        ra = lm.RouteArgs(T=T, E=E, k=k, logits=fake, topk_ids=fake, topk_w=fake, sorted_row=fake, row_pos=fake,
                          offsets=fake, workspace=ws, workspace_bytes=0 if ws is None else 1 << 30)
        fa = lm.ForwardArgs(d=d, l=l, I=I, S=S, Is=Is, wfmt=0, norm_eps=1e-6, x=fake, w_in=fake, w1=fake, w3=fake,
                            w2=fake, norm_w=fake, w_out=fake, ws1=fake, ws3=fake, ws2=fake, y=fake)
        return ra, fa
    ra, fa = args(T, ws=fake)
    with pytest.raises(lm.LatentMoeError) as ei:
        lm.latent_moe_layer_noalloc(ra, None, None, fa)
    assert ei.value.code == lm.LMOE_EINVAL
    big = 4096
    need = (lm.route_workspace_size(big, E, k) + 255) // 256 * 256 + lm.forward_workspace_size(big, E, k, d, l, I,
                                                                                            S, Is)
    assert need > lm.NOALLOC_SCRATCH_BYTES
    ra, fa = args(big)
    with pytest.raises(lm.LatentMoeError) as ei:
        lm.latent_moe_layer_noalloc(ra, None, None, fa)
    assert ei.value.code == lm.LMOE_EUNSUPPORTED
    assert "scratch" in str(ei.value)


def test_output_stationary_layer_refusals():
    """latent_moe_layer_os refuses what it does not serve before any HIP call
    (no GPU needed; the stand-in pointers are never read)."""
    import latentmoe_expert_layer_amd as lm
    fake = 1 << 20
    ws_big = 1 << 40

    def args(T=256, E=896, k=16, l=256, I=256, wfmt=0, logits=True):
        ra = lm.RouteArgs(T=T, E=E, k=k, logits=fake if logits else None, ids_in=None if logits else fake,
                          weights_in=None if logits else fake, topk_ids=fake, topk_w=fake)
        fa = lm.ForwardArgs(d=512, l=l, I=I, S=2, Is=256, wfmt=wfmt, norm_eps=1e-6, x=fake, w_in=fake, w1=fake,
                            w3=fake, w2=fake, s1=fake, s3=fake, s2=fake, norm_w=fake, w_out=fake, ws1=fake,
                            ws3=fake, ws2=fake, y=fake, workspace=fake, workspace_bytes=ws_big)
        return ra, fa
    cases = [(dict(logits=False, k=1), lm.LMOE_EINVAL),
             (dict(T=600), lm.LMOE_EUNSUPPORTED),                  # beyond a decode batch
             (dict(T=512, k=17, E=896), lm.LMOE_EUNSUPPORTED),     # T*k > 8192
             (dict(wfmt=lm.LMOE_WFMT_MXFP4), lm.LMOE_EUNSUPPORTED),
             (dict(wfmt=lm.LMOE_WFMT_MXFP4_W4A16, l=384), lm.LMOE_EUNSUPPORTED),
             (dict(l=192, I=128), lm.LMOE_EUNSUPPORTED)]
    for kw, code in cases:
        ra, fa = args(**kw)
        with pytest.raises(lm.LatentMoeError) as ei:
            lm.latent_moe_layer_os(ra, fa)
        assert ei.value.code == code, (kw, ei.value)


def test_tile_packed_layout_refusals():
    """The tile-packed weight layout is refused where no kernel reads it, and
    the pack call validates its arguments, before any HIP call (no GPU)."""
    import latentmoe_expert_layer_amd as lm
    fake = 1 << 20
    ws_big = 1 << 40

    def fwd(wfmt=0, l=256, I=256, wlayout=lm.LMOE_WLAYOUT_TILED):
        return lm.ForwardArgs(d=512, l=l, I=I, S=2, Is=256, wfmt=wfmt, norm_eps=1e-6, x=fake, w_in=fake, w1=fake,
                              w3=fake, w2=fake, s1=fake, s3=fake, s2=fake, norm_w=fake, w_out=fake, ws1=fake,
                              ws3=fake, ws2=fake, y=fake, workspace=fake, workspace_bytes=ws_big, wlayout=wlayout)
    ra = lm.RouteArgs(T=256, E=896, k=16, logits=fake, topk_ids=fake, topk_w=fake)
    for kw, code in [(dict(wfmt=lm.LMOE_WFMT_MXFP4), lm.LMOE_EUNSUPPORTED),
                     (dict(l=192, I=256), lm.LMOE_EUNSUPPORTED),
                     (dict(l=256, I=128), lm.LMOE_EUNSUPPORTED),
                     (dict(wlayout=7), lm.LMOE_EINVAL)]:
        with pytest.raises(lm.LatentMoeError) as ei:
            lm.latent_moe_layer_os(ra, fwd(**kw))
        assert ei.value.code == code, kw
    for args in [(fake, fake, 2, 100, 64), (fake, fake, 2, 128, 96), (fake, fake + 8, 1, 128, 64),
                 (fake, fake + 1024, 4, 128, 64)]:   # N, K not multiples; misaligned; overlapping
        with pytest.raises(lm.LatentMoeError) as ei:
            lm.latent_moe_pack_weights(*args)
        assert ei.value.code == lm.LMOE_EINVAL, args

