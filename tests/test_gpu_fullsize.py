"""GPU parity at the full workload sizes, in the launch configuration the benchmark
times. Each workload's layer runs once on the GPU and its results are kept on the host;
then the oracle checks EVERY expert, one expert (or, for the 128-expert workload, one
group of experts) per test, and a last test per workload checks every token after the
GPU's combine.

  * routing indices and the permutation: bit-exact for all tokens;
  * bf16 outputs: max|a-b| / max|b| <= 2e-2 per expert and over all tokens;
  * MXFP8 and per-tensor FP8 outputs: <= 6e-2 against the oracle's
    quantise/dequantise reference (per-tensor FP8: one test over all rows, since a
    tensor's factor spans every expert);
  * backward: y, dx and dprob rows and both weight gradients of every expert; dx and the
    GPU's dprob gather ([T, k], the gradient w.r.t. the routing probabilities) over all
    tokens.
"""
import numpy as np
import pytest
import torch

import oracle
from conftest import max_rel_err, record_parity
from gpu_util import bf16_bits, dev_bf16, dev_f32
from moe_inputs import WORKLOADS, bf16_bits_to_f32, make_inputs

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

BF16_TOL = 2e-2
MX_TOL = 6e-2
FP8_TOL = 6e-2


@pytest.fixture(scope="module")
def moe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import grouped_expert_gemm_amd as g
    g.lib()
    return g


_INPUTS = {}   # the last workload's inputs (one slot: the Mixtral weights are 2.8 GB of bits)
_RUNS = {}     # GPU results on the host, per workload run


def _inputs(name):
    w = WORKLOADS[name]
    key = (w.seed, w.T, w.H, w.I, w.E, w.k, w.zipf, w.backward)
    if key not in _INPUTS:
        _INPUTS.clear()
        _INPUTS[key] = make_inputs(w, want_float=False)
    return _INPUTS[key]


def _h32(t):
    """Device tensor -> float32 numpy (bf16 through its bits, exactly)."""
    if t.dtype == torch.bfloat16:
        return bf16_bits_to_f32(bf16_bits(t))
    return t.detach().cpu().numpy().astype(np.float32)


def _done_with_gpu():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _route_and_permute(moe, inp, w):
    idx, p = moe.moe_route_topk(dev_f32(inp.logits), w.k)
    r = moe.moe_permute(dev_bf16(inp.bits["x"]), idx, p, w.E)
    torch.cuda.synchronize()
    # routing indices and the whole permutation are graded bit-exact
    ridx, rp = oracle.route_topk(inp.logits, w.k)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    m = oracle.permute(ridx, w.E)
    for key in ("split_sizes", "offsets", "row_id_map", "src_token"):
        assert np.array_equal(r[key].cpu().numpy(), m[key]), key
    pp = rp.ravel()[m["src_token"] * w.k + m["src_slot"]]
    return idx, r, m, pp


def _expert(run, e):
    """Rows [a, b) of expert e, its x rows (float32), routing weights and weights."""
    inp, m, pp = run["inp"], run["m"], run["pp"]
    a, b = int(m["offsets"][e]), int(m["offsets"][e + 1])
    x = bf16_bits_to_f32(inp.bits["x"][m["src_token"][a:b]])
    W1 = bf16_bits_to_f32(inp.bits["w1"][e:e + 1])
    W2 = bf16_bits_to_f32(inp.bits["w2"][e:e + 1])
    return a, b, x, pp[a:b], W1, W2


# ---------------------------------------------------------------------------
# forward workloads: Mixtral bf16, Qwen3 bf16 (skewed, idle experts), Mixtral MXFP8
# ---------------------------------------------------------------------------

def _forward_run(moe, name):
    if name in _RUNS:
        return _RUNS[name]
    _RUNS.clear()
    w = WORKLOADS[name]
    inp = _inputs(name)
    compute = "mxfp8" if w.dtype == "mxfp8" else "bf16"
    print(f"{name}: T={w.T} H={w.H} I={w.I} E={w.E} k={w.k} ({compute}), GPU layer", flush=True)
    idx, r, m, pp = _route_and_permute(moe, inp, w)
    if name == "qwen3_fwd":
        assert (np.diff(m["offsets"]) == 0).any(), "the skewed workload must leave experts idle"
    w1, w2 = dev_bf16(inp.bits["w1"]), dev_bf16(inp.bits["w2"])
    y = moe.moe_grouped_mlp_fwd(r["x_perm"], w1, w2, r["offsets"], r["prob_perm"], compute=compute)
    out = moe.moe_unpermute_combine(y, r["row_id_map"], w.T, w.k)
    run = dict(w=w, inp=inp, m=m, pp=pp, tol=MX_TOL if compute == "mxfp8" else BF16_TOL, y=_h32(y), out=_h32(out),
               ref_y={})
    del idx, r, w1, w2, y, out
    _done_with_gpu()
    _RUNS[name] = run
    return run


def _ref_forward(run, e):
    if e not in run["ref_y"]:
        a, b, x, pe, W1, W2 = _expert(run, e)
        if run["w"].dtype == "mxfp8":
            ref, _ = oracle.grouped_mlp_forward_mxfp8(x, W1, W2, np.array([0, b - a]), pe)
        else:
            ref, _, _ = oracle.grouped_mlp_forward(x, W1, W2, np.array([0, b - a]), pe)
        run["ref_y"][e] = ref
    return run["ref_y"][e]


FWD_CASES = ([("mixtral_fwd", (e,)) for e in range(8)]
             + [("qwen3_fwd", tuple(range(16 * g, 16 * g + 16))) for g in range(8)]
             + [("mixtral_mxfp8_fwd", (e,)) for e in range(8)])


@pytest.mark.parametrize("name,experts", FWD_CASES,
                         ids=[f"{n}-e{x[0]}" + (f"-{x[-1]}" if len(x) > 1 else "") for n, x in FWD_CASES])
def test_forward_full_size_experts(moe, name, experts):
    run = _forward_run(moe, name)
    for e in experts:
        a, b = int(run["m"]["offsets"][e]), int(run["m"]["offsets"][e + 1])
        if a == b:
            print(f"  expert {e}: no rows", flush=True)
            continue
        err = max_rel_err(run["y"][a:b], _ref_forward(run, e))
        print(f"  expert {e}: rows {b - a}, y max rel err {err:.2e}", flush=True)
        record_parity(f"full size {name} per expert", y=err)
        assert err <= run["tol"], e


@pytest.mark.parametrize("name", ["mixtral_fwd", "qwen3_fwd", "mixtral_mxfp8_fwd"])
def test_forward_full_size_combine(moe, name):
    """Every token's output after the GPU combine, against the oracle's combine of the
    oracle's per-expert results."""
    run = _forward_run(moe, name)
    w, m = run["w"], run["m"]
    ref_y = np.zeros((w.R, w.H))
    for e in range(w.E):
        a, b = int(m["offsets"][e]), int(m["offsets"][e + 1])
        if b > a:
            ref_y[a:b] = _ref_forward(run, e)
    ref_out = oracle.unpermute_combine(ref_y, m["row_id_map"], w.T, w.k)
    err = max_rel_err(run["out"], ref_out)
    print(f"{name}: out over all {w.T} tokens, max rel err {err:.2e}", flush=True)
    record_parity(f"full size {name} all tokens", out=err)
    assert err <= run["tol"]
    _RUNS.clear()


# ---------------------------------------------------------------------------
# Mixtral forward + backward (T = 4096), bf16
# ---------------------------------------------------------------------------

def _fwd_bwd_run(moe):
    name = "mixtral_fwd_bwd/bf16"
    if name in _RUNS:
        return _RUNS[name]
    _RUNS.clear()
    w = WORKLOADS["mixtral_fwd_bwd"]
    inp = _inputs("mixtral_fwd_bwd")
    print(f"mixtral_fwd_bwd: T={w.T} H={w.H} I={w.I}, GPU layer forward + backward (bf16)", flush=True)
    idx, r, m, pp = _route_and_permute(moe, inp, w)
    w1, w2 = dev_bf16(inp.bits["w1"]), dev_bf16(inp.bits["w2"])
    y, z, h = moe.moe_grouped_mlp_fwd(r["x_perm"], w1, w2, r["offsets"], r["prob_perm"], save_for_bwd=True)
    out = moe.moe_unpermute_combine(y, r["row_id_map"], w.T, w.k)
    dyp = moe.moe_permute(dev_bf16(inp.bits["dout"]), idx, None, w.E, row_id_map=r["row_id_map"])["x_perm"]
    dxp, dw1, dw2, dprob = moe.moe_grouped_mlp_bwd(dyp, r["x_perm"], z, h, r["prob_perm"], w1, w2, r["offsets"])
    dx = moe.moe_unpermute_combine(dxp, r["row_id_map"], w.T, w.k)
    # the gradient w.r.t. the routing probabilities: dprob[t, j] = dprob_perm[row_id_map[t*k + j]],
    # gathered on the GPU as a one-slot combine of one-column rows
    dprob_tk = moe.moe_unpermute_combine(dprob.view(w.R, 1), r["row_id_map"], w.R, 1).view(w.T, w.k)
    run = dict(w=w, inp=inp, m=m, pp=pp, y=_h32(y), out=_h32(out), dxp=_h32(dxp), dx=_h32(dx),
               dprob_perm=dprob.cpu().numpy(), dprob=dprob_tk.cpu().numpy(), dw1=bf16_bits(dw1), dw2=bf16_bits(dw2),
               ref={})
    del idx, r, w1, w2, y, z, h, out, dyp, dxp, dw1, dw2, dprob, dx, dprob_tk
    _done_with_gpu()
    _RUNS[name] = run
    return run


def _ref_fwd_bwd(run, e):
    if e not in run["ref"]:
        a, b, x, pe, W1, W2 = _expert(run, e)
        dy = bf16_bits_to_f32(run["inp"].bits["dout"][run["m"]["src_token"][a:b]])
        y, _, _ = oracle.grouped_mlp_forward(x, W1, W2, np.array([0, b - a]), pe)
        g = oracle.grouped_mlp_backward(dy, x, W1, W2, np.array([0, b - a]), pe)
        run["ref"][e] = dict(y=y, dx_perm=g["dx_perm"], dprob_perm=g["dprob_perm"], dw1=g["dw_gate_up"][0],
                             dw2=g["dw_down"][0])
    return run["ref"][e]


@pytest.mark.parametrize("e", range(8))
def test_forward_backward_full_size_expert(moe, e):
    run = _fwd_bwd_run(moe)
    a, b = int(run["m"]["offsets"][e]), int(run["m"]["offsets"][e + 1])
    ref = _ref_fwd_bwd(run, e)
    errs = {
        "y": max_rel_err(run["y"][a:b], ref["y"]),
        "dx_perm": max_rel_err(run["dxp"][a:b], ref["dx_perm"]),
        "dprob": max_rel_err(run["dprob_perm"][a:b], ref["dprob_perm"]),
        "dw_gate_up": max_rel_err(bf16_bits_to_f32(run["dw1"][e]), ref["dw1"]),
        "dw_down": max_rel_err(bf16_bits_to_f32(run["dw2"][e]), ref["dw2"]),
    }
    print(f"  expert {e}: rows {b - a}, " + ", ".join(f"{k} {v:.2e}" for k, v in errs.items()), flush=True)
    record_parity("full size mixtral_fwd_bwd bf16 per expert", **errs)
    for k, v in errs.items():
        assert v <= BF16_TOL, k


def test_forward_backward_full_size_tokens(moe):
    """out, dx (after the GPU combine) and dprob [T, k] (the GPU gather) for every token."""
    run = _fwd_bwd_run(moe)
    w, m = run["w"], run["m"]
    ref_y = np.zeros((w.R, w.H))
    ref_dxp = np.zeros((w.R, w.H))
    ref_dprob = np.zeros(w.R)
    for e in range(w.E):
        a, b = int(m["offsets"][e]), int(m["offsets"][e + 1])
        ref = _ref_fwd_bwd(run, e)
        ref_y[a:b], ref_dxp[a:b], ref_dprob[a:b] = ref["y"], ref["dx_perm"], ref["dprob_perm"]
    errs = {
        "out": max_rel_err(run["out"], oracle.unpermute_combine(ref_y, m["row_id_map"], w.T, w.k)),
        "dx": max_rel_err(run["dx"], oracle.unpermute_combine(ref_dxp, m["row_id_map"], w.T, w.k)),
        "dprob": max_rel_err(run["dprob"], ref_dprob[m["row_id_map"]].reshape(w.T, w.k)),
    }
    print(f"mixtral_fwd_bwd all {w.T} tokens: " + ", ".join(f"{k} {v:.2e}" for k, v in errs.items()), flush=True)
    record_parity("full size mixtral_fwd_bwd bf16 all tokens", **errs)
    for k, v in errs.items():
        assert v <= BF16_TOL, k
    # the gather itself moves bits: dprob[t, j] is exactly the GPU's dprob_perm of its row
    assert np.array_equal(run["dprob"].ravel(), run["dprob_perm"][m["row_id_map"]])
    _RUNS.clear()


# ---------------------------------------------------------------------------
# Mixtral forward + backward (T = 4096), grouped MLP in MXFP8
# ---------------------------------------------------------------------------

def _mx_fwd_bwd_run(moe):
    name = "mixtral_fwd_bwd/mxfp8"
    if name in _RUNS:
        return _RUNS[name]
    _RUNS.clear()
    w = WORKLOADS["mixtral_fwd_bwd"]
    inp = _inputs("mixtral_fwd_bwd")
    print(f"mixtral_fwd_bwd: T={w.T} H={w.H} I={w.I}, GPU layer forward + backward (MXFP8)", flush=True)
    idx, r, m, pp = _route_and_permute(moe, inp, w)
    w1, w2 = dev_bf16(inp.bits["w1"]), dev_bf16(inp.bits["w2"])
    y, z, h = moe.moe_grouped_mlp_fwd(r["x_perm"], w1, w2, r["offsets"], r["prob_perm"], compute="mxfp8",
                                      save_for_bwd=True)
    dyp = moe.moe_permute(dev_bf16(inp.bits["dout"]), idx, None, w.E, row_id_map=r["row_id_map"])["x_perm"]
    dxp, dw1, dw2, dprob = moe.moe_grouped_mlp_bwd(dyp, r["x_perm"], z, h, r["prob_perm"], w1, w2, r["offsets"],
                                                   compute="mxfp8")
    dx = moe.moe_unpermute_combine(dxp, r["row_id_map"], w.T, w.k)
    run = dict(w=w, inp=inp, m=m, pp=pp, y=_h32(y), z=bf16_bits(z), h=bf16_bits(h), dxp=_h32(dxp), dx=_h32(dx),
               dprob_perm=dprob.cpu().numpy(), dw1=bf16_bits(dw1), dw2=bf16_bits(dw2), ref={})
    del idx, r, w1, w2, y, z, h, dyp, dxp, dw1, dw2, dprob, dx
    _done_with_gpu()
    _RUNS[name] = run
    return run


@pytest.mark.parametrize("e", range(8))
def test_mxfp8_forward_backward_full_size_expert(moe, e):
    """Expert e of the MXFP8 training step: y, and the saved z and h, against the
    oracle's MXFP8 forward; dx, dprob, dW1, dW2 (the GPU backward ran on the GPU's saved
    z and h) against the oracle's MXFP8 backward on the oracle forward's own z and h
    rounded to bf16, both with the bf16 roundings of dH and dZ that the recipe's return
    to bf16 implies and without them."""
    run = _mx_fwd_bwd_run(moe)
    a, b, x, pe, W1, W2 = _expert(run, e)
    offs = np.array([0, b - a])
    y, h_ref, z_ref = oracle.grouped_mlp_forward_mxfp8(x, W1, W2, offs, pe, return_z=True)
    fwd = {"y": max_rel_err(run["y"][a:b], y), "z": max_rel_err(bf16_bits_to_f32(run["z"][a:b]), z_ref),
           "h": max_rel_err(bf16_bits_to_f32(run["h"][a:b]), h_ref)}
    dy = bf16_bits_to_f32(run["inp"].bits["dout"][run["m"]["src_token"][a:b]])
    zs, hs = oracle.bf16_round(z_ref), oracle.bf16_round(h_ref)
    got = {"dx_perm": run["dxp"][a:b], "dprob_perm": run["dprob_perm"][a:b],
           "dw_gate_up": bf16_bits_to_f32(run["dw1"][e]), "dw_down": bf16_bits_to_f32(run["dw2"][e])}
    errs = {}
    for rounded in (True, False):
        g = oracle.grouped_mlp_backward_mxfp8(dy, x, zs, hs, W1, W2, offs, pe, round_bf16=rounded)
        for k in got:
            errs[(k, rounded)] = max_rel_err(got[k], g[k] if k == "dx_perm" or k == "dprob_perm" else g[k][0])
        if rounded:
            run["ref"][e] = dict(dx_perm=g["dx_perm"])
    print(f"  expert {e}: rows {b - a}, " + ", ".join(f"{k} {v:.2e}" for k, v in fwd.items()) + "; "
          + ", ".join(f"{k} {v:.2e}/{errs[(k, False)]:.2e}" for (k, r), v in errs.items() if r)
          + " (with/without the dH, dZ bf16 roundings)", flush=True)
    record_parity("full size mixtral_fwd_bwd MXFP8 forward per expert", **fwd)
    record_parity("full size mixtral_fwd_bwd MXFP8 backward per expert, dH/dZ rounded to bf16",
                  **{k: v for (k, r), v in errs.items() if r})
    record_parity("full size mixtral_fwd_bwd MXFP8 backward per expert, no dH/dZ rounding",
                  **{k: v for (k, r), v in errs.items() if not r})
    assert fwd["y"] <= MX_TOL and fwd["z"] <= 1e-2 and fwd["h"] <= 1e-2
    for (k, rounded), v in errs.items():
        assert v <= MX_TOL, (k, rounded)


def test_mxfp8_forward_backward_full_size_tokens(moe):
    """dx after the GPU combine for every token of the MXFP8 training step."""
    run = _mx_fwd_bwd_run(moe)
    w, m = run["w"], run["m"]
    ref_dxp = np.zeros((w.R, w.H))
    for e in range(w.E):
        a, b, x, pe, W1, W2 = _expert(run, e)
        if e not in run["ref"]:
            offs = np.array([0, b - a])
            dy = bf16_bits_to_f32(run["inp"].bits["dout"][m["src_token"][a:b]])
            _, h_ref, z_ref = oracle.grouped_mlp_forward_mxfp8(x, W1, W2, offs, pe, return_z=True)
            g = oracle.grouped_mlp_backward_mxfp8(dy, x, oracle.bf16_round(z_ref), oracle.bf16_round(h_ref), W1, W2,
                                                  offs, pe)
            run["ref"][e] = dict(dx_perm=g["dx_perm"])
        ref_dxp[a:b] = run["ref"][e]["dx_perm"]
    err = max_rel_err(run["dx"], oracle.unpermute_combine(ref_dxp, m["row_id_map"], w.T, w.k))
    print(f"mixtral_fwd_bwd MXFP8: dx over all {w.T} tokens, max rel err {err:.2e}", flush=True)
    record_parity("full size mixtral_fwd_bwd MXFP8 all tokens", dx=err)
    assert err <= MX_TOL
    _RUNS.clear()
    _INPUTS.clear()


# ---------------------------------------------------------------------------
# Mixtral forward + backward (T = 4096), grouped MLP in per-tensor FP8
# ---------------------------------------------------------------------------

def test_fp8_forward_backward_full_size(moe):
    """The per-tensor FP8 training step at the full Mixtral fwd+bwd size, every expert
    and every token: y, the saved z and h against the oracle's FP8 forward over all rows;
    dx (per row and after the GPU combine), dprob, dW1, dW2 (the GPU backward ran on the
    GPU's saved z and h) against the oracle's FP8 backward on the oracle forward's own z
    (rounded to bf16) and bf16 h, with dH and dZ rounded to bf16 (the reading without
    those roundings is checked at the small shapes of test_gpu_fp8_bwd.py). One factor
    per tensor spans all experts, so the oracle runs on all rows at once."""
    w = WORKLOADS["mixtral_fwd_bwd"]
    inp = _inputs("mixtral_fwd_bwd")
    _RUNS.clear()
    print(f"mixtral_fwd_bwd: T={w.T} H={w.H} I={w.I}, GPU layer forward + backward (per-tensor FP8)", flush=True)
    idx, r, m, pp = _route_and_permute(moe, inp, w)
    w1, w2 = dev_bf16(inp.bits["w1"]), dev_bf16(inp.bits["w2"])
    y, z, h = moe.moe_grouped_mlp_fwd(r["x_perm"], w1, w2, r["offsets"], r["prob_perm"], compute="fp8",
                                      save_for_bwd=True)
    dyp = moe.moe_permute(dev_bf16(inp.bits["dout"]), idx, None, w.E, row_id_map=r["row_id_map"])["x_perm"]
    dxp, dw1, dw2, dprob = moe.moe_grouped_mlp_bwd(dyp, r["x_perm"], z, h, r["prob_perm"], w1, w2, r["offsets"],
                                                   compute="fp8")
    dx = moe.moe_unpermute_combine(dxp, r["row_id_map"], w.T, w.k)
    got = dict(y=_h32(y), z=_h32(z), h=_h32(h), dx_perm=_h32(dxp), dx=_h32(dx), dprob_perm=dprob.cpu().numpy(),
               dw_gate_up=_h32(dw1), dw_down=_h32(dw2))
    del idx, r, w1, w2, y, z, h, dyp, dxp, dw1, dw2, dprob, dx
    _done_with_gpu()
    off, src = m["offsets"], m["src_token"]
    x = bf16_bits_to_f32(inp.bits["x"][src])
    W1, W2 = bf16_bits_to_f32(inp.bits["w1"]), bf16_bits_to_f32(inp.bits["w2"])
    y_ref, z_ref, h_ref = oracle.grouped_mlp_forward_fp8_tensor(x, W1, W2, off, pp, return_zh=True)
    fwd = {"y": max_rel_err(got["y"], y_ref), "z": max_rel_err(got["z"], z_ref), "h": max_rel_err(got["h"], h_ref)}
    print("  forward " + ", ".join(f"{k} {v:.2e}" for k, v in fwd.items()), flush=True)
    dy = bf16_bits_to_f32(inp.bits["dout"][src])
    g = oracle.grouped_mlp_backward_fp8_tensor(dy, x, oracle.bf16_round(z_ref), h_ref, W1, W2, off, pp)
    errs = {k: max_rel_err(got[k], g[k]) for k in ("dx_perm", "dprob_perm", "dw_gate_up", "dw_down")}
    errs["dx"] = max_rel_err(got["dx"], oracle.unpermute_combine(g["dx_perm"], m["row_id_map"], w.T, w.k))
    for e in range(w.E):   # every expert's weight gradients on their own scale
        errs[f"dw_gate_up[{e}]"] = max_rel_err(got["dw_gate_up"][e], g["dw_gate_up"][e])
        errs[f"dw_down[{e}]"] = max_rel_err(got["dw_down"][e], g["dw_down"][e])
    print("  backward " + ", ".join(f"{k} {v:.2e}" for k, v in errs.items() if "[" not in k)
          + f"; worst expert dW1 {max(v for k, v in errs.items() if k.startswith('dw_gate_up[')):.2e}, "
          f"dW2 {max(v for k, v in errs.items() if k.startswith('dw_down[')):.2e}", flush=True)
    record_parity("full size mixtral_fwd_bwd FP8 forward", **fwd)
    record_parity("full size mixtral_fwd_bwd FP8 backward, dH/dZ rounded to bf16",
                  **{k: v for k, v in errs.items() if "[" not in k})
    assert fwd["y"] <= FP8_TOL and fwd["z"] <= 1e-2 and fwd["h"] <= 1e-2
    for k, v in errs.items():
        assert v <= FP8_TOL, k
    _INPUTS.clear()
