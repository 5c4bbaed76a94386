"""Pins for the CPU oracle: checks against things other than the oracle itself.

Each test compares the oracle with an independent definition (brute force on
tiny inputs, a library routine, a closed form, a published table), chosen so
that a dropped term, a wrong sign or index, or a transposed operand anywhere in
``oracle/oracle.cpp`` fails at least one of them.  No GPU is used.
"""
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def bf16(t):
    """Round to bf16 (library cast, nearest-even) and back to float64."""
    return torch.as_tensor(t).to(torch.float32).to(torch.bfloat16).to(torch.float64)


def read_table(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                a, b = line.split()
                rows.append((a, b))
    return rows


# ------------------------------------------------------------------ codecs
def test_e2m1_table_matches_ocp():
    for code, val in read_table("e2m1_values.txt"):
        got = oracle.e2m1_value(int(code))
        assert got == float(val) and math.copysign(1, got) == math.copysign(1, float(val)), code


def test_e8m0_all_codes():
    for c in range(255):
        assert oracle.e8m0_value(c) == 2.0 ** (c - 127)
    assert math.isnan(oracle.e8m0_value(255))


def test_e4m3_decode_matches_torch_float8_e4m3fn():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float32)
    for c in range(256):
        got = oracle.e4m3_value(c)
        r = ref[c].item()
        if math.isnan(r):
            assert math.isnan(got), c
        else:
            assert got == r and math.copysign(1, got) == math.copysign(1, r), c


def test_e4m3_encode_matches_torch_cast():
    rng = np.random.default_rng(3)
    vals = list(rng.standard_normal(4000) * 60.0) + list(rng.standard_normal(1000) * 0.01)
    # every exact midpoint between consecutive finite codes (ties go to the even code)
    pos = [oracle.e4m3_value(c) for c in range(0x7F)]
    vals += [(a + b) / 2 for a, b in zip(pos[:-1], pos[1:])]
    vals += [-v for v in vals[-126:]] + [0.0, -0.0, 448.0, 449.0, 463.9, 470.0, 1e6, -1e6, 2.0 ** -10]
    t = torch.tensor(vals, dtype=torch.float32)
    ref = t.clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8)
    for v, r in zip(t.tolist(), ref.tolist()):
        got = oracle.e4m3_encode(v)
        if r & 0x7F == 0:  # zero: sign of zero is immaterial for the product
            assert got & 0x7F == 0, v
        else:
            assert got == r, (v, got, r)


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(5)
    vals = rng.standard_normal(3000).astype(np.float32)
    bits = rng.integers(0, 2**32, 2000, dtype=np.uint64).astype(np.uint32).view(np.float32)
    bits = bits[np.isfinite(bits)]
    # exact ties: low 16 bits == 0x8000
    ties = (rng.integers(0, 2**16, 500, dtype=np.uint32) << 16 | 0x8000).astype(np.uint32).view(np.float32)
    ties = ties[np.isfinite(ties)]
    allv = np.concatenate([vals, bits, ties])
    ref = torch.from_numpy(allv).to(torch.bfloat16).view(torch.int16).numpy().astype(np.uint16)
    for v, r in zip(allv.tolist(), ref.tolist()):
        assert oracle.to_bf16_bits(v) == r, v
    assert oracle.to_bf16_bits(float("nan")) & 0x7FC0 == 0x7FC0


def ref_mxfp8(v):
    """OCP MX v1.0 MXFP8 conversion via torch: X = 2^(floor(log2 amax) - 8),
    elements = float8_e4m3fn(clamp(v / X))."""
    v = torch.as_tensor(v, dtype=torch.float32).view(-1, 32)
    amax = v.abs().amax(dim=1)
    _, e = torch.frexp(amax)
    sexp = torch.where(amax > 0, (e - 1 - 8).clamp(-127, 127), torch.full_like(e, -127))
    scaled = torch.ldexp(v, -sexp[:, None].to(torch.float32))
    q = scaled.clamp(-448, 448).to(torch.float8_e4m3fn)
    deq = q.to(torch.float32) * torch.pow(2.0, sexp.to(torch.float32))[:, None]
    return deq.view(-1), q.view(torch.uint8).view(-1), (sexp + 127).to(torch.uint8)


def test_mxfp8_non_finite_blocks_and_extreme_scales():
    """Reading: a block holding a NaN or an infinity quantises to the NaN
    block (e8m0 255 = NaN, every e4m3fn code 0x7F = NaN); finite blocks at
    the ends of bf16's range get the shared exponent floor(log2 amax) - 8
    clamped to e8m0's range, as the torch reference computes it."""
    g = torch.Generator().manual_seed(13)
    v = torch.randn(8 * 32, generator=g)
    v[3] = float("nan")                       # block 0: one NaN
    v[32 + 31] = float("inf")                 # block 1: +inf
    v[64] = float("-inf")                     # block 2: -inf
    v[96:128] = float("nan")                  # block 3: all NaN
    v[128:160] = (torch.rand(32, generator=g) * 2 - 1) * 3.0e38  # block 4: near bf16 max (3.39e38)
    v[128] = 3.0e38
    v[160:192] = torch.randn(32, generator=g) * 2.0 ** -130  # block 5: bf16 subnormals
    v = v.to(torch.bfloat16).float()
    deq, codes, scales = oracle.mxfp8(v)
    for b in range(4):
        assert scales[b].item() == 255, b
        assert torch.all(codes[32 * b:32 * b + 32] == 0x7F), b
        assert torch.all(torch.isnan(deq[32 * b:32 * b + 32])), b
    fin = slice(128, 256)
    rdeq, rcodes, rscales = ref_mxfp8(v[fin])
    assert torch.equal(scales[4:], rscales)
    nz = rcodes & 0x7F != 0
    assert torch.equal(codes[fin][nz], rcodes[nz])
    assert torch.equal(deq[fin], rdeq)
    assert scales[4].item() == 127 + 127 - 8       # amax in [2^127, 2^128)
    assert scales[5].item() == 0                   # floor(log2 amax) - 8 below -127: clamped
    assert oracle.e4m3_encode(float("nan")) & 0x7F == 0x7F


def test_mxfp8_block_quantisation_matches_reference():
    g = torch.Generator().manual_seed(11)
    v = torch.randn(64 * 32, generator=g) * torch.logspace(-3, 3, 64).repeat_interleave(32)
    v[:32] = 0.0                                  # all-zero block
    v[32:64] = 0.25                               # amax exactly a power of two
    v[64:96] = torch.randn(32, generator=g) * 1e-30  # tiny block
    deq, codes, scales = oracle.mxfp8(v)
    rdeq, rcodes, rscales = ref_mxfp8(v)
    assert torch.equal(scales, rscales)
    nz = rcodes & 0x7F != 0
    assert torch.equal(codes[nz], rcodes[nz])
    assert torch.all(codes[~nz] & 0x7F == 0)
    assert torch.equal(deq, rdeq)


# ------------------------------------------------------------------ router
def brute_topk(logits, k):
    """Rank by (value desc, index asc) with NaN last, via Python's sort."""
    out = []
    for row in logits.tolist():
        key = lambda e: (1, 0.0, e) if math.isnan(row[e]) else (0, -row[e], e)
        out.append(sorted(range(len(row)), key=key)[:k])
    return torch.tensor(out, dtype=torch.int32)


@pytest.mark.parametrize("T,E,k", [(64, 16, 4), (9, 896, 16), (33, 56, 1), (5, 7, 7)])
def test_route_ids_brute_force(T, E, k):
    logits = W.separated_logits(0, f"r{T}", T, E, k)
    ids, w = oracle.route(logits, k)
    assert torch.equal(ids, brute_topk(logits, k))
    # weights: library softmax over the selected logits, float64
    sel = torch.gather(logits.double(), 1, ids.long())
    ref = torch.softmax(sel, dim=1)
    assert torch.allclose(w.double(), ref, atol=2e-6, rtol=0)
    assert torch.allclose(w.double().sum(1), torch.ones(T, dtype=torch.float64), atol=1e-5)


def test_route_ties_nan_and_signed_zero():
    # quantised logits: many exact ties; the lower index must win
    g = torch.Generator().manual_seed(2)
    logits = (torch.randn(40, 24, generator=g) * 4).round() / 4
    logits[0, :] = 1.0                      # all equal -> first k indices, weights 1/k
    logits[1, :] = float("nan")             # all NaN -> first k indices
    logits[2, :5] = float("nan")            # NaNs rank below every number
    logits[3, :] = -1.0
    logits[3, 7] = -0.0
    logits[3, 3] = 0.0                      # +0 == -0: index 3 before 7
    ids, w = oracle.route(logits, 6)
    assert torch.equal(ids, brute_topk(logits, 6))
    assert torch.equal(ids[0], torch.arange(6, dtype=torch.int32))
    assert torch.allclose(w[0], torch.full((6,), 1 / 6))
    assert ids[3, 0] == 3 and ids[3, 1] == 7
    assert not any(int(e) < 5 for e in ids[2])


def test_route_weight_ratio_closed_form():
    logits = torch.full((1, 10), -50.0)
    logits[0, 4] = 1.0
    logits[0, 8] = 1.0 - 0.7
    ids, w = oracle.route(logits, 2)
    assert ids.tolist() == [[4, 8]]
    assert abs(w[0, 0].item() / w[0, 1].item() - math.exp(0.7)) < 1e-5


# ----------------------------------------------------------------- permute
def test_permute_rejects_out_of_range_ids():
    for bad in ([0, 3, 4], [-1, 0, 2]):
        with pytest.raises(ValueError):
            oracle.permute(torch.tensor(bad, dtype=torch.int32), 4)


@pytest.mark.parametrize("R,E", [(256, 16), (4096, 896), (1000, 56), (7, 3), (0, 5)])
def test_permute_invariants_and_stable_sort(R, E):
    g = torch.Generator().manual_seed(R + E)
    ids = torch.randint(0, E, (R,), generator=g, dtype=torch.int32)
    if R > 10:
        ids[: R // 3] = E - 1                   # one heavy expert, others possibly empty
    offsets, sorted_row, row_pos = oracle.permute(ids, E)
    counts = torch.bincount(ids.long(), minlength=E)
    assert offsets[0] == 0 and torch.equal(offsets[1:].long() - offsets[:-1].long(), counts)
    # library stable sort defines the unique stable permutation
    ref = torch.from_numpy(np.argsort(ids.numpy(), kind="stable").astype(np.int32))
    assert torch.equal(sorted_row, ref)
    assert torch.equal(row_pos[sorted_row.long()], torch.arange(R, dtype=torch.int32))


# ------------------------------------------------------------ whole layer
def dense_reference(inp, k, act_quant=False, norm=True):
    """Brute force: evaluate EVERY expert on EVERY token in float64 (bf16 at the
    storage points), mask with the token's top-k, weight and sum."""
    cfg = inp["cfg"]
    f = lambda n: inp[n].to(torch.float64)
    if cfg.mxfp4:
        table = torch.tensor([float(v) for _, v in read_table("e2m1_values.txt")], dtype=torch.float64)

        def deq(codes, scales, N, K):
            c = codes.view(cfg.E, N, K // 2).long()
            lo, hi = c & 15, c >> 4
            el = torch.stack([table[lo], table[hi]], dim=-1).view(cfg.E, N, K)
            sc = torch.pow(2.0, scales.view(cfg.E, N, K // 32).double() - 127)
            return el * sc.repeat_interleave(32, dim=2)

        W1, W3 = deq(inp["w1q"], inp["s1"], cfg.I, cfg.l), deq(inp["w3q"], inp["s3"], cfg.I, cfg.l)
        W2 = deq(inp["w2q"], inp["s2"], cfg.l, cfg.I)
    else:
        W1, W3, W2 = f("w1"), f("w3"), f("w2")
    aq = (lambda v: ref_mxfp8(v.float())[0].double().view(v.shape)) if act_quant else (lambda v: v)
    x = f("x")
    if cfg.rows_mode:
        z = x
        gates = torch.zeros(cfg.T, cfg.E, dtype=torch.float64)
        gates[torch.arange(cfg.T), inp["ids"].view(-1).long()] = inp["weights"].view(-1).double()
    else:
        z = bf16(x @ f("w_in").T)
        # router gate on the latent (float64), or the given logits
        logits = z @ f("w_r").T if "w_r" in inp else inp["logits"]
        sel = brute_topk(logits, k).long()
        wsel = torch.softmax(torch.gather(logits.double(), 1, sel), dim=1)
        gates = torch.zeros(cfg.T, cfg.E, dtype=torch.float64)
        gates.scatter_(1, sel, wsel)
    za = aq(z)
    c = torch.zeros(cfg.T, cfg.l, dtype=torch.float64)
    for e in range(cfg.E):
        H = bf16(F.silu(za @ W1[e].T) * (za @ W3[e].T))
        Y = bf16(aq(H) @ W2[e].T)
        c += gates[:, e:e + 1] * Y
    if cfg.rows_mode:
        return bf16(c)
    if norm and "norm_w" in inp:
        rh = bf16(c / torch.sqrt((c * c).mean(dim=1, keepdim=True) + cfg.eps) * f("norm_w"))
    else:
        rh = bf16(c)
    y = rh @ f("w_out").T
    for s in range(cfg.S):
        hs = bf16(F.silu(x @ f("ws1")[s].T) * (x @ f("ws3")[s].T))
        y = y + hs @ f("ws2")[s].T
    return bf16(y)


def assert_close(got, ref, max_rel=2e-2, mae=1e-3):
    got, ref = got.double(), ref.double()
    floor = 0.1 * ref.pow(2).mean().sqrt()
    rel = (got - ref).abs() / torch.maximum(ref.abs(), floor)
    assert rel.max().item() <= max_rel, rel.max().item()
    assert (got - ref).abs().mean().item() <= mae, (got - ref).abs().mean().item()


SMALL = [
    dict(T=13, d=96, l=64, E=6, k=3, S=2, I=32, Is=48),
    dict(T=20, d=64, l=96, E=5, k=2, S=1, I=64, Is=32),
    dict(T=9, d=128, l=64, E=4, k=4, S=0, I=96, Is=0),      # k = E: dense softmax mixture
]


@pytest.mark.parametrize("dims", SMALL)
@pytest.mark.parametrize("norm", ["ones", "random", "none"])
@pytest.mark.parametrize("korder", [0, 1])
def test_layer_matches_dense_brute_force(dims, norm, korder):
    """korder 1 (every K reduction descending, the second valid order used to
    measure the tolerance) is pinned the same way."""
    cfg = W.custom(**dims)
    inp = W.make_inputs(cfg, norm_w=norm)
    out = oracle.run(inp, korder=korder)
    ref = dense_reference(inp, cfg.k)
    assert_close(out["y"], ref, max_rel=1e-2, mae=2e-4)


def test_layer_intermediates_layout():
    cfg = W.custom(T=11, d=64, l=64, E=5, k=2, S=1, I=32, Is=32)
    inp = W.make_inputs(cfg)
    out = oracle.run(inp, intermediates=True)
    x = inp["x"].double()
    assert torch.equal(out["z"].double(), bf16(x @ inp["w_in"].double().T))
    # H/Y are in sorted order: position p holds row sorted_row[p] = t*k + j
    for p in range(cfg.T * cfg.k):
        r = int(out["sorted_row"][p])
        t, e = r // cfg.k, int(out["ids"].view(-1)[r])
        zt = out["z"][t].double()
        h = bf16(F.silu(zt @ inp["w1"][e].double().T) * (zt @ inp["w3"][e].double().T))
        assert (out["H"][p].double() - h).abs().max() <= 1e-2 * h.abs().max()
    # sampled-token evaluation equals the full evaluation
    sub = oracle.run(inp, eval_tokens=[3, 0, 10])
    assert torch.equal(sub["y"], out["y"][[3, 0, 10]])


def test_textbook_swiglu_special_case():
    # E = k = 1, S = 0, d = l, W_in = W_out = identity, no norm: y = SwiGLU(x)
    cfg = W.custom(T=16, d=64, l=64, E=1, k=1, S=0, I=96, Is=0, norm=False)
    inp = W.make_inputs(cfg)
    eye = torch.eye(64, dtype=torch.bfloat16)
    inp["w_in"], inp["w_out"] = eye, eye
    out = oracle.run(inp)
    x = inp["x"].double()
    H = bf16(F.silu(x @ inp["w1"][0].double().T) * (x @ inp["w3"][0].double().T))
    ref = bf16(H @ inp["w2"][0].double().T)
    assert_close(out["y"], ref, max_rel=1e-2, mae=1e-4)


def test_zero_expert_down_proj_leaves_shared_only():
    cfg = W.custom(T=10, d=96, l=64, E=6, k=3, S=2, I=32, Is=48)
    inp = W.make_inputs(cfg)
    inp["w2"] = torch.zeros_like(inp["w2"])
    out = oracle.run(inp)
    x = inp["x"].double()
    y = torch.zeros(cfg.T, cfg.d, dtype=torch.float64)
    for s in range(cfg.S):
        hs = bf16(F.silu(x @ inp["ws1"][s].double().T) * (x @ inp["ws3"][s].double().T))
        y += hs @ inp["ws2"][s].double().T
    assert_close(out["y"], bf16(y), max_rel=1e-2, mae=1e-4)


def test_identical_experts_make_routing_irrelevant():
    cfg = W.custom(T=12, d=64, l=64, E=5, k=2, S=1, I=32, Is=32)
    inp = W.make_inputs(cfg)
    for n in ("w1", "w3", "w2"):
        inp[n] = inp[n][:1].expand_as(inp[n]).contiguous()
    a = oracle.run(inp)["y"]
    inp["logits"] = W.separated_logits(7, "other", cfg.T, cfg.E, cfg.k)
    b = oracle.run(inp)["y"]
    assert_close(a, b, max_rel=1e-2, mae=1e-4)


def test_rows_mode_matches_dense_brute_force():
    cfg = W.custom(T=300, d=0, l=64, E=7, k=1, S=0, I=32, Is=0, rows_mode=True, norm=False, zipf_s=1.1)
    inp = W.make_inputs(cfg)
    out = oracle.run(inp)
    assert_close(out["y"], dense_reference(inp, 1), max_rel=1e-2, mae=1e-4)


@pytest.mark.parametrize("act_quant", [True, False])
def test_mxfp4_layer_matches_dense_brute_force(act_quant):
    cfg = W.custom(T=10, d=96, l=64, E=5, k=2, S=1, I=64, Is=32, mxfp4=True)
    inp = W.make_inputs(cfg)
    out = oracle.run(inp, act_quant=act_quant)
    ref = dense_reference(inp, cfg.k, act_quant=act_quant)
    # a flipped bf16 rounding of an input to the MXFP8 quantiser can move one
    # element by one e4m3 step (1/8 relative), hence the looser bound here
    assert_close(out["y"], ref, max_rel=5e-2, mae=2e-3)


# ----------------------------------------------------------- router gate
def test_router_logits_integer_exact():
    """Small-integer operands make every product and partial sum exact in fp32,
    so the logits must equal integer matrix products bit for bit: a transposed
    gate, a wrong row or a dropped term changes them."""
    g = torch.Generator().manual_seed(5)
    T, d, l, E = 11, 64, 96, 40
    x = torch.randint(-2, 3, (T, d), generator=g)
    w_in = torch.randint(-2, 3, (l, d), generator=g)
    w_r = torch.randint(-3, 4, (E, l), generator=g)
    zi = x.long() @ w_in.long().T                   # |z| <= 256: exact in bf16
    logits, z = oracle.router_logits(x.to(torch.bfloat16), w_in.to(torch.bfloat16), w_r.to(torch.bfloat16))
    assert torch.equal(z.to(torch.int64), zi)
    assert torch.equal(logits.to(torch.int64), zi @ w_r.long().T)
    assert torch.equal(logits, logits.round())
    # the latent given directly (no down-projection)
    l2, z2 = oracle.router_logits(zi.to(torch.bfloat16), None, w_r.to(torch.bfloat16))
    assert torch.equal(l2, logits) and torch.equal(z2, z)


def test_router_logits_score_the_rounded_latent():
    """The gate reads z after its bf16 rounding: latents 257 and 259 (not bf16
    values) are scored as 256 and 260 (round to nearest, ties to even)."""
    d, l, E = 64, 64, 64
    x = torch.zeros(2, d)
    x[0, 0], x[0, 1] = 256.0, 1.0
    x[1, 0], x[1, 1] = 256.0, 3.0
    w_in = torch.zeros(l, d)
    w_in[0, 0] = w_in[0, 1] = 1.0
    w_in[1, 0] = 1.0
    w_in[1, 1] = 1.0
    eye = torch.eye(E, l)
    logits, z = oracle.router_logits(x.to(torch.bfloat16), w_in.to(torch.bfloat16), eye.to(torch.bfloat16))
    assert logits[0, :2].tolist() == [256.0, 256.0]
    assert logits[1, :2].tolist() == [260.0, 260.0]
    assert torch.equal(logits[:, 2:], torch.zeros(2, E - 2))


def separate_latent_routing(inp, min_gap=1e-3, rounds=100):
    """Redraw x rows until every token's float64 latent logits have their k+1
    largest values at least min_gap apart (the fp32 rounding of the oracle then
    cannot reorder them)."""
    cfg = inp["cfg"]
    for r in range(rounds):
        z = bf16(inp["x"].double() @ inp["w_in"].double().T)
        top = torch.topk(z @ inp["w_r"].double().T, cfg.k + 1, dim=1).values
        bad = ((top[:, :-1] - top[:, 1:]) < min_gap).any(dim=1).nonzero().flatten()
        if bad.numel() == 0:
            return inp
        inp["x"][bad] = W.normal_bf16(cfg.seed, f"x.redraw{r}", (bad.numel(), cfg.d), 1.0)
    raise RuntimeError("could not separate the latent router logits")


@pytest.mark.parametrize("dims", SMALL[:2])
def test_layer_with_router_gate_matches_dense_brute_force(dims):
    cfg = W.custom(router_gemm=True, **dims)
    inp = separate_latent_routing(W.make_inputs(cfg))
    out = oracle.run(inp)
    ref = dense_reference(inp, cfg.k)
    assert_close(out["y"], ref, max_rel=1e-2, mae=2e-4)
    # the oracle's logits are the float64 gate products up to fp32 rounding
    z = bf16(inp["x"].double() @ inp["w_in"].double().T)
    assert (out["logits"].double() - z @ inp["w_r"].double().T).abs().max() < 1e-5


def test_page_moe_shape():
    facts = dict((a, int(b)) for a, b in read_table("moe_shape.txt"))
    cfg = W.CONFIGS["prefill"]
    assert (cfg.E, cfg.k, cfg.S) == (facts["routed_experts"], facts["top_k"], facts["shared_experts"])
    dec = W.CONFIGS["decode"]
    assert (dec.d, dec.l) == (facts["latent_example_in"], facts["latent_example_out"])
    logits = W.separated_logits(0, "shape", 4, facts["routed_experts"], facts["top_k"])
    ids, w = oracle.route(logits, facts["top_k"])
    for row in ids.tolist():
        assert len(set(row)) == facts["top_k"]
        assert all(0 <= e < facts["routed_experts"] for e in row)
