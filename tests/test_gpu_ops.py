"""GPU parity of each C-ABI entry point against the CPU oracle, at sizes that span
several tiles with ragged tails, plus edge cases (empty experts, one expert
taking every token, T = 1, k = E). Integer and byte outputs must match exactly;
floating outputs within the stated tolerances (max|a-b| / max|b|)."""
import numpy as np
import pytest
import torch

import oracle
from conftest import max_rel_err
from moe_inputs import WORKLOADS, f32_to_bf16_bits, bf16_bits_to_f32, make_inputs, scaled

pytestmark = pytest.mark.gpu

BF16_TOL = 2e-2     # bf16 outputs with float32 accumulation
PROB_TOL = 1e-6     # float32 routing weights


@pytest.fixture(scope="module")
def moe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import grouped_expert_gemm_amd as g
    g.lib()
    return g


from gpu_util import bf16_bits, dev_bf16, dev_f32, host, oracle_perm  # noqa: E402


# ---------------------------------------------------------------------------
# router
# ---------------------------------------------------------------------------

def _route_case(moe, logits, k, renorm=True):
    idx, p = moe.moe_route_topk(dev_f32(logits), k, renorm)
    ridx, rp = oracle.route_topk(logits, k, renorm)
    print(f"route T={logits.shape[0]} E={logits.shape[1]} k={k}", flush=True)
    assert np.array_equal(idx.cpu().numpy(), ridx), "top-k indices differ"
    np.testing.assert_allclose(p.cpu().numpy(), rp, rtol=PROB_TOL, atol=1e-7)


@pytest.mark.parametrize("name", ["tiny", "qwen3_fwd", "mixtral_fwd"])
def test_route_workloads(moe, name):
    w = WORKLOADS[name]
    inp = make_inputs(scaled(w, H=32, I=32, E=w.E), want_float=False)  # logits do not depend on H, I
    _route_case(moe, inp.logits, w.k)


def test_route_edges(moe):
    rng = np.random.default_rng(0)
    ties = np.round(rng.standard_normal((333, 16))).astype(np.float32)   # many exact ties
    _route_case(moe, ties, 4)
    _route_case(moe, rng.standard_normal((1, 8)).astype(np.float32), 2)  # T = 1
    _route_case(moe, rng.standard_normal((100, 6)).astype(np.float32), 6)  # k = E
    _route_case(moe, rng.standard_normal((100, 256)).astype(np.float32), 16)
    _route_case(moe, rng.standard_normal((77, 32)).astype(np.float32), 3, renorm=False)
    # every lane-group width: E = 1, 3 (a group of 4 with an empty lane), 65 and 200
    # (two and four logits per lane, partly empty), odd token counts
    _route_case(moe, rng.standard_normal((5, 1)).astype(np.float32), 1)
    _route_case(moe, rng.standard_normal((37, 3)).astype(np.float32), 2)
    _route_case(moe, rng.standard_normal((129, 65)).astype(np.float32), 7, renorm=False)
    _route_case(moe, np.round(2 * rng.standard_normal((61, 200))).astype(np.float32), 9)
    # -inf logits are ranked like any number (ties among them by index)
    neg = rng.standard_normal((50, 16)).astype(np.float32)
    neg[:, 3:] = -np.inf
    _route_case(moe, neg, 5)


# ---------------------------------------------------------------------------
# permutation and combine
# ---------------------------------------------------------------------------

def _permute_case(moe, T, H, E, k, idx, p, dtype="bf16"):
    rng = np.random.default_rng(T + E)
    xf = rng.standard_normal((T, H)).astype(np.float32)
    xb = f32_to_bf16_bits(xf)
    x = dev_bf16(xb) if dtype == "bf16" else dev_f32(xf)
    r = moe.moe_permute(x, torch.from_numpy(idx.astype(np.int32)).cuda(), dev_f32(p), E)
    m = oracle.permute(idx, E)
    print(f"permute T={T} H={H} E={E} k={k}", flush=True)
    for key in ("split_sizes", "offsets", "row_id_map", "src_token"):
        assert np.array_equal(r[key].cpu().numpy(), m[key]), key
    pp = p.ravel()[m["src_token"] * k + m["src_slot"]].astype(np.float32)
    assert np.array_equal(r["prob_perm"].cpu().numpy(), pp)
    if dtype == "bf16":
        assert np.array_equal(bf16_bits(r["x_perm"]), xb[m["src_token"]])
    else:
        assert np.array_equal(r["x_perm"].cpu().numpy(), xf[m["src_token"]])
    return r, m, x


def test_permute_workloads(moe):
    for name in ("tiny", "qwen3_fwd"):
        w = WORKLOADS[name]
        inp = make_inputs(scaled(w, H=32, I=32), want_float=False)
        idx, p = oracle.route_topk(inp.logits, w.k)
        sizes = np.bincount(idx.ravel(), minlength=w.E)
        if name == "qwen3_fwd":
            assert (sizes == 0).any()
        _permute_case(moe, w.T, 256, w.E, w.k, idx, p.astype(np.float32))


def test_permute_edges(moe):
    rng = np.random.default_rng(1)
    # every token to expert 3 (k = 1), the others empty
    idx = np.full((1000, 1), 3, np.int32)
    _permute_case(moe, 1000, 64, 8, 1, idx, np.ones((1000, 1), np.float32))
    # T = 1, k = E
    idx, p = oracle.route_topk(rng.standard_normal((1, 5)).astype(np.float32), 5)
    _permute_case(moe, 1, 40, 5, 5, idx, p.astype(np.float32))
    # odd row width (byte-wise copies), float32 rows, many blocks
    idx, p = oracle.route_topk(rng.standard_normal((2049, 256)).astype(np.float32), 16)
    _permute_case(moe, 2049, 3, 256, 16, idx, p.astype(np.float32), dtype="f32")
    # block counts over more than one LDS chunk of the scan (E = 256: 32 block rows per chunk)
    idx, p = oracle.route_topk(rng.standard_normal((9000, 256)).astype(np.float32), 2)
    _permute_case(moe, 9000, 16, 256, 2, idx, p.astype(np.float32))
    # an expert count that does not divide the scan's 256 threads
    idx, p = oracle.route_topk(rng.standard_normal((3000, 200)).astype(np.float32), 3)
    _permute_case(moe, 3000, 16, 200, 3, idx, p.astype(np.float32))


def test_permute_drops_repeated_and_out_of_range_ids(moe):
    """The input contract of moe_permute: a (token, slot) pair whose expert id is out of
    [0, E) or repeats an earlier slot's id is dropped (row -1, not counted); the rest
    are permuted exactly as if the dropped pairs were absent, and the combine skips them."""
    rng = np.random.default_rng(3)
    T, H, E, k = 1100, 64, 8, 3
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    idx[rng.choice(T, 60, replace=False), 2] = idx[:, 0][rng.choice(T, 60, replace=False)]  # some repeats
    rep = rng.choice(T, 40, replace=False)
    idx[rep, 2] = idx[rep, 1]                                                                   # repeats
    bad = rng.choice(T, 40, replace=False)
    idx[bad, 1] = rng.choice([-1, -7, E, E + 3, 1 << 30], 40)                                 # out of range
    keep = np.ones_like(idx, bool)
    for j in range(k):
        keep[:, j] &= (idx[:, j] >= 0) & (idx[:, j] < E)
        for i in range(j):
            keep[:, j] &= idx[:, j] != idx[:, i]
    assert (~keep).sum() > 50
    clean = np.where(keep, idx, -1)
    p = rng.uniform(0.1, 1, (T, k)).astype(np.float32)
    xb = f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    print(f"permute with dropped pairs: T={T} E={E} k={k}, {(~keep).sum()} dropped", flush=True)
    r = moe.moe_permute(dev_bf16(xb), torch.from_numpy(idx).cuda(), dev_f32(p), E)
    m = oracle.permute(clean, E)
    n = int(m["offsets"][E])
    assert n == keep.sum()
    for key in ("split_sizes", "offsets", "row_id_map"):
        assert np.array_equal(r[key].cpu().numpy(), m[key]), key
    assert np.array_equal(r["src_token"].cpu().numpy()[:n], m["src_token"][:n])
    assert np.array_equal(bf16_bits(r["x_perm"])[:n], xb[m["src_token"][:n]])
    pp = p.ravel()[m["src_token"][:n] * k + m["src_slot"][:n]]
    assert np.array_equal(r["prob_perm"].cpu().numpy()[:n], pp)
    # the combine adds only the kept pairs of each token
    yh = rng.standard_normal((n, H)).astype(np.float32)
    y = torch.zeros((T * k, H), dtype=torch.float32, device="cuda")
    y[:n] = torch.from_numpy(yh).cuda()
    out = moe.moe_unpermute_combine(y, r["row_id_map"], T, k).cpu().numpy()
    ref = oracle.unpermute_combine(np.concatenate([yh, np.zeros((1, H), np.float32)]),
                                   np.where(m["row_id_map"] < 0, n, m["row_id_map"]), T, k)
    assert np.abs(out - ref).max() <= 1e-6 * np.abs(ref).max()


def test_permute_reuse_map_and_mxfp8_rows(moe):
    rng = np.random.default_rng(2)
    T, H, E, k = 777, 128, 8, 2
    idx, p = oracle.route_topk(rng.standard_normal((T, E)).astype(np.float32), k)
    r, m, _ = _permute_case(moe, T, H, E, k, idx, p.astype(np.float32))
    g = f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    out = moe.moe_permute(dev_bf16(g), torch.from_numpy(idx).cuda(), None, E, row_id_map=r["row_id_map"])
    assert np.array_equal(bf16_bits(out["x_perm"]), g[m["src_token"]])
    codes = torch.from_numpy(rng.integers(0, 255, (T, H), dtype=np.uint8)).cuda()
    sc = torch.from_numpy(rng.integers(0, 255, (T, H // 32), dtype=np.uint8)).cuda()
    q = moe.moe_permute(codes, torch.from_numpy(idx).cuda(), dev_f32(p), E, x_scale=sc)
    assert np.array_equal(q["x_perm"].cpu().numpy(), codes.cpu().numpy()[m["src_token"]])
    assert np.array_equal(q["x_perm_scale"].cpu().numpy(), sc.cpu().numpy()[m["src_token"]])


@pytest.mark.parametrize("T,H,E,k", [(700, 1096, 16, 6), (300, 2048, 128, 8), (129, 8, 4, 3)])
def test_combine_shapes(moe, T, H, E, k):
    """bf16 combine: row widths with a partial last group of chunks per lane, slot counts
    with a partial group of four slots, weighted and unweighted."""
    rng = np.random.default_rng(T + H + k)
    idx, p = oracle.route_topk(rng.standard_normal((T, E)).astype(np.float32), k)
    m = oracle.permute(idx, E)
    yb = f32_to_bf16_bits(rng.standard_normal((T * k, H)).astype(np.float32))
    rmap = torch.from_numpy(m["row_id_map"].astype(np.int32)).cuda()
    print(f"combine T={T} H={H} k={k}", flush=True)
    out = moe.moe_unpermute_combine(dev_bf16(yb), rmap, T, k)
    ref = oracle.unpermute_combine(bf16_bits_to_f32(yb), m["row_id_map"], T, k)
    assert max_rel_err(host(out), ref) <= 2.0 ** -8
    outw = moe.moe_unpermute_combine(dev_bf16(yb), rmap, T, k, dev_f32(p.astype(np.float32)))
    refw = oracle.unpermute_combine(bf16_bits_to_f32(yb), m["row_id_map"], T, k, weights=p)
    assert max_rel_err(host(outw), refw) <= 2.0 ** -8
    # permutation of the same rows: bit-exact gather into each of the k rows
    xb = f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    r = moe.moe_permute(dev_bf16(xb), torch.from_numpy(idx.astype(np.int32)).cuda(),
                        dev_f32(p.astype(np.float32)), E)
    assert np.array_equal(bf16_bits(r["x_perm"]), xb[m["src_token"]])


def test_combine(moe):
    rng = np.random.default_rng(3)
    T, H, E, k = 1500, 512, 8, 2
    idx, p = oracle.route_topk(rng.standard_normal((T, E)).astype(np.float32), k)
    m = oracle.permute(idx, E)
    yb = f32_to_bf16_bits(rng.standard_normal((T * k, H)).astype(np.float32))
    rmap = torch.from_numpy(m["row_id_map"].astype(np.int32)).cuda()
    out = moe.moe_unpermute_combine(dev_bf16(yb), rmap, T, k)
    ref = oracle.unpermute_combine(bf16_bits_to_f32(yb), m["row_id_map"], T, k)
    assert max_rel_err(host(out), ref) <= 2.0 ** -8
    outw = moe.moe_unpermute_combine(dev_bf16(yb), rmap, T, k, dev_f32(p.astype(np.float32)))
    refw = oracle.unpermute_combine(bf16_bits_to_f32(yb), m["row_id_map"], T, k, weights=p)
    assert max_rel_err(host(outw), refw) <= 2.0 ** -8
    # k = 1, unit weights: the inverse permutation, bit for bit
    idx1, _ = oracle.route_topk(rng.standard_normal((T, E)).astype(np.float32), 1)
    m1 = oracle.permute(idx1, E)
    xb = f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    back = moe.moe_unpermute_combine(dev_bf16(xb[m1["src_token"]]),
                                     torch.from_numpy(m1["row_id_map"].astype(np.int32)).cuda(), T, 1)
    assert np.array_equal(bf16_bits(back), xb)
    # float32 rows, odd width
    yf = rng.standard_normal((T * k, 7)).astype(np.float32)
    outf = moe.moe_unpermute_combine(dev_f32(yf), rmap, T, k)
    np.testing.assert_allclose(outf.cpu().numpy(), oracle.unpermute_combine(yf, m["row_id_map"], T, k),
                               rtol=1e-6, atol=1e-6)


def test_combine_rounds_to_nearest_bf16(moe):
    """The kernels round a float32 result to bf16 once, to nearest with ties to even (the
    packed conversion of gfx950). With k = 1 and weights of at most 16 significant bits,
    every product w * y of a bf16 value y is exact in float32, so the combine's output is
    that one rounding of the exact product: it must equal the oracle's bf16 rounding bit
    for bit. Half of the rows hold powers of two, which the weights 1 + 2^-8, 1 + 3 2^-8,
    1 + 5 2^-8 put exactly half-way between two bf16 values, and 1 + 2^-8 -+ 2^-16 just
    below and above; the other rows are normal draws times 16-bit weights."""
    rng = np.random.default_rng(11)
    T, H = 1024, 256
    y = rng.standard_normal((T, H)).astype(np.float32)
    pw = rng.choice([-1.0, 1.0], size=(T // 2, H)) * np.exp2(rng.integers(-20, 21, size=(T // 2, H)))
    y[: T // 2] = pw
    yb = f32_to_bf16_bits(y)
    w_ties = [1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, 1 + 5 * 2.0 ** -8, 1 + 2.0 ** -8 - 2.0 ** -16,
              1 + 2.0 ** -8 + 2.0 ** -16, 1 - 2.0 ** -9, 0.75 + 2.0 ** -10, -(1 + 2.0 ** -8)]
    w = np.empty(T)
    for t in range(T):
        if t < T // 2:
            w[t] = w_ties[t % len(w_ties)]
        else:  # 16 significant bits
            w[t] = rng.integers(1 << 15, 1 << 16) * 2.0 ** (-15 + int(rng.integers(-3, 4))) * rng.choice([-1.0, 1.0])
    assert np.all(w.astype(np.float32).astype(np.float64) == w)
    exact = bf16_bits_to_f32(yb).astype(np.float64) * w[:, None]
    ref = oracle.bf16_round(exact)
    # how many products sit exactly half-way between two bf16 values (the case that
    # tells round-half-even from other rules)
    e = np.floor(np.log2(np.abs(exact)))
    frac = np.abs(exact) / np.exp2(e - 7)
    ties = int(np.sum(frac - np.floor(frac) == 0.5))
    assert ties > 1000, ties
    rmap = torch.arange(T, dtype=torch.int32).cuda()
    print(f"combine rounding T={T} H={H} ties={ties}", flush=True)
    out = moe.moe_unpermute_combine(dev_bf16(yb), rmap, T, 1, dev_f32(w.astype(np.float32)))
    assert np.array_equal(bf16_bits(out), f32_to_bf16_bits(ref.astype(np.float32)))


# ---------------------------------------------------------------------------
# MXFP8 quantisation: bit-exact
# ---------------------------------------------------------------------------

COLWISE = [
    # name, expert sizes, C, pad
    ("ragged_idle", [37, 0, 100, 1, 162], 128, 32),
    ("gemm_pad", [300, 5, 0, 257], 64, 256),
    ("odd_blocks", [130, 0, 260, 7], 192, 32),   # three 64-column blocks: item pairs straddle row groups
    ("mixtral_bwd_dY", None, 4096, 256),   # the T=4096 backward's dY: 8192 rows, 8 experts
]


@pytest.mark.parametrize("case", COLWISE, ids=[c[0] for c in COLWISE])
def test_mxfp8_quantize_colwise_bit_exact(moe, case):
    name, sizes, C, pad = case
    rng = np.random.default_rng(21)
    if sizes is None:
        w = WORKLOADS["mixtral_fwd_bwd"]
        idx, _ = oracle.route_topk(make_inputs(scaled(w, H=32, I=32), want_float=False).logits, w.k)
        sizes = list(np.bincount(idx.ravel(), minlength=w.E))
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    R = int(off[-1])
    xb = f32_to_bf16_bits((rng.standard_normal((R, C)) * np.exp2(rng.integers(-6, 6, (R, 1)))).astype(np.float32))
    print(f"mxfp8 colwise {name}: R={R} C={C} E={len(sizes)} pad={pad}", flush=True)
    codes, scales, kofs = moe.mxfp8_quantize_colwise(dev_bf16(xb), torch.from_numpy(off).cuda(), pad)
    torch.cuda.synchronize()
    kcap = codes.shape[1]
    rc, rs, rk = oracle.mxfp8_quantize_colwise(bf16_bits_to_f32(xb), off, pad, kcap)
    assert np.array_equal(kofs.cpu().numpy(), rk)
    assert np.array_equal(codes.cpu().numpy(), rc)
    assert np.array_equal(scales.cpu().numpy(), rs)


def test_mxfp8_quantize_colwise_special_values(moe):
    """Blocks along the token axis holding zeros, negative zeros, bf16 subnormals, a block
    whose maximum sits on a scale boundary, values near the top of the float range, values
    below 2^-126, one large value over ones (the rest land on subnormal codes) and a
    ramp through zero; three experts, the middle one empty."""
    rng = np.random.default_rng(3)
    R, C = 320, 128
    x = rng.standard_normal((R, C)).astype(np.float32)
    x *= np.exp2(rng.integers(-40, 40, (R // 32, C))).repeat(32, 0).astype(np.float32)
    x[0:32, 0] = 0.0
    x[32:64, 1] = -0.0
    x[64:96, 2] = rng.standard_normal(32) * 1e-39
    x[96:128, 3] = 448.0 * 2.0 ** 5
    x[128:160, 4] = rng.standard_normal(32) * 3e38 / 4
    x[160:192, 5] = rng.standard_normal(32) * 2.0 ** -130
    x[192:224, 6] = 1.0
    x[192, 6] = 2.0 ** 20
    x[224:256, 7] = np.linspace(-1, 1, 32) * 2.0 ** -7
    xb = f32_to_bf16_bits(x)
    off = np.array([0, 100, 100, 320], np.int32)
    codes, scales, kofs = moe.mxfp8_quantize_colwise(dev_bf16(xb), torch.from_numpy(off).cuda(), 32)
    torch.cuda.synchronize()
    rc, rs, rk = oracle.mxfp8_quantize_colwise(bf16_bits_to_f32(xb), off, 32, codes.shape[1])
    assert np.array_equal(kofs.cpu().numpy(), rk)
    assert np.array_equal(codes.cpu().numpy(), rc)
    assert np.array_equal(scales.cpu().numpy(), rs)


def test_mxfp8_quantize_bit_exact(moe):
    rng = np.random.default_rng(4)
    rows, cols = 300, 1024
    x = rng.standard_normal((rows, cols)).astype(np.float32)
    x *= np.exp2(rng.integers(-40, 40, (rows, cols // 32))).repeat(32, 1).astype(np.float32)
    x[5, 64:96] = 0.0                                       # zero block
    x[6, :32] = -0.0                                        # negative zeros
    x[7, 32:64] = rng.standard_normal(32) * 1e-39           # bf16 subnormals
    x[8, 64:96] = 448.0 * 2.0 ** 5                          # exactly on the scale boundary
    x[9, :] = rng.standard_normal(cols) * 3e38 / 4          # near the top of the range
    xb = f32_to_bf16_bits(x)
    codes, scales = moe.mxfp8_quantize(dev_bf16(xb))
    rc, rs = oracle.mxfp8_quantize(bf16_bits_to_f32(xb))
    assert np.array_equal(scales.cpu().numpy(), rs)
    assert np.array_equal(codes.cpu().numpy(), rc)


def test_mxfp8_quantize_weight_shape(moe):
    """A Mixtral gate_up weight slice: one expert's first 2048 rows x 4096."""
    w = WORKLOADS["mixtral_fwd"]
    g = np.random.default_rng(np.random.SeedSequence(w.seed).spawn(6)[1])
    xb = f32_to_bf16_bits(np.float32(0.02) * g.standard_normal((2048, 4096), np.float32))
    codes, scales = moe.mxfp8_quantize(dev_bf16(xb))
    rc, rs = oracle.mxfp8_quantize(bf16_bits_to_f32(xb))
    assert np.array_equal(scales.cpu().numpy(), rs)
    assert np.array_equal(codes.cpu().numpy(), rc)

