"""GPU parity of the backward pass against the CPU oracle
(oracle/backward_oracle.py): a whole training step (forward with the
pre-activations kept, then every backward call through the C ABI) on seeded
workloads, compared output by output; fp32 layers within 1e-5 and bf16 layers
within 1e-2 (max|err| / max|ref|), as the forward."""
import numpy as np
import pytest
import torch

import routing_dispatch_expert_moe_amd as M
from oracle import backward_oracle as B
from oracle import moe_oracle as O
from workloads import custom, make, output_grad

from gpu_util import DEV, as64, capacity_of, log, t_in, t_out, weights_fn

pytestmark = pytest.mark.gpu


def upload(wl, chunk=8, keep_host=False):
    """Forward operands (packed w13, w2p) and backward operands (w13_t [E,d,2f],
    w2_t = W2 [E,f,d]) of the workload's local experts, built on the GPU."""
    tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    E_loc, d, f = wl.E_loc, wl.d, wl.f
    w13 = torch.empty((E_loc, 2 * f, d), dtype=tdt, device=DEV)
    w2p = torch.empty((E_loc, d, f), dtype=tdt, device=DEV)
    w13_t = torch.empty((E_loc, d, 2 * f), dtype=tdt, device=DEV)
    w2_t = torch.empty((E_loc, f, d), dtype=tdt, device=DEV)
    host = [] if keep_host else None
    for c0 in range(0, E_loc, chunk):
        ids = list(range(wl.e_begin + c0, wl.e_begin + min(E_loc, c0 + chunk)))
        a, b, c = wl.stacked_weights(ids)
        if keep_host:
            host.extend(zip(a, b, c))
        n = len(ids)
        ga, gb = t_in(a, wl.dtype), t_in(b, wl.dtype)
        w2_t[c0:c0 + n] = t_in(c, wl.dtype)
        M.moe_pack_weights(ga, gb, w2_t[c0:c0 + n], w13[c0:c0 + n], w2p[c0:c0 + n])
        M.moe_pack_weights_backward(ga, gb, w13_t[c0:c0 + n])
    torch.cuda.synchronize()
    return w13, w2p, w13_t, w2_t, host


def train_step(wl, ops, C, logits=None):
    """Forward (route, dispatch, up with pre-activations, down, combine) and the
    whole backward through the C ABI.  Returns every tensor by name."""
    w13, w2p, w13_t, w2_t = ops
    T, E, k = wl.T, wl.E, wl.k
    x = t_in(wl.x, wl.dtype)
    out = {}
    if logits is None:
        if wl.logits is not None:
            logits = torch.from_numpy(wl.logits).to(DEV)
        else:
            wg = torch.from_numpy(wl.w_gate).to(DEV)
            logits = M.moe_router_logits(x, wg)
            out["w_gate"] = wg
    ws = M.alloc_workspace(T, E, k, wl.E_loc)
    idx, w = M.moe_route(logits, k, wl.gate)
    plan = M.moe_dispatch(idx, E, C, wl.e_begin, wl.e_end, x, ws)
    rows = plan.max_rows
    h, ab = M.moe_ffn_up_train(plan.x_perm, plan.offsets, wl.E_loc, rows, w13)
    y_perm = M.moe_ffn_down(h, plan.offsets, wl.E_loc, rows, w2p)
    y = M.moe_combine(y_perm, plan.pair_pos, w)
    dy = t_in(output_grad(wl), wl.dtype)
    do_perm, dgate = M.moe_combine_backward(dy, y_perm, plan.pair_pos, w)
    dlogits = M.moe_gate_backward(logits, idx, dgate, wl.gate)
    dh, dab = M.moe_ffn_down_backward(do_perm, plan.offsets, wl.E_loc, rows, w2_t, ab)
    dx_perm = M.moe_ffn_up_backward(dab, plan.offsets, wl.E_loc, rows, w13_t)
    dx = M.moe_combine(dx_perm, plan.pair_pos, None, T=T, k=k)
    dw13, dw2 = M.moe_ffn_wgrad(plan.x_perm, h, do_perm, dab, plan.offsets, wl.E_loc, rows)
    if "w_gate" in out:
        dx, out["dw_gate"] = M.moe_router_backward(x, out["w_gate"], dlogits, dx)
    torch.cuda.synchronize()
    assert M.moe_check_error(ws) == 0
    out.update(logits=logits, idx=idx, w=w, plan=plan, h=h, ab=ab, y_perm=y_perm, y=y,
               do_perm=do_perm, dgate=dgate, dlogits=dlogits, dh=dh, dab=dab, dx_perm=dx_perm,
               dx=dx, dw13=dw13, dw2=dw2)
    return out


def check_against_oracle(wl, g, tol, host=None):
    f = wl.f
    logits_f32 = t_out(g["logits"])
    wg64 = O.widen(wl.w_gate, "f32") if wl.w_gate is not None else None
    ref = B.moe_layer_backward(wl.x, wl.dtype, logits_f32, wl.k, wl.gate, weights_fn(wl, host),
                               wl.E, output_grad(wl), capacity_of(wl), wl.e_begin, wl.e_end,
                               w_gate64=wg64)
    fwd = ref["fwd"]
    n = int(np.asarray(fwd["offsets"])[-1])
    assert np.array_equal(t_out(g["plan"].pair_pos)[:wl.T * wl.k], fwd["pair_pos"])
    assert np.array_equal(t_out(g["plan"].offsets), fwd["offsets"])
    dt = wl.dtype
    errs = {}
    ab = as64(g["ab"][:n], dt)   # rows past n_kept are never written
    errs["a"] = O.rel_err(ab[:, :f], ref["a"]) if n else 0.0
    errs["g"] = O.rel_err(ab[:, f:], ref["g"]) if n else 0.0
    errs["h"] = O.rel_err(as64(g["h"][:n], dt), ref["h"]) if n else 0.0
    errs["do_perm"] = O.rel_err(as64(g["do_perm"][:n], dt), ref["do_perm"])
    errs["dgate"] = O.rel_err(t_out(g["dgate"]), ref["dgate"])
    errs["dlogits"] = O.rel_err(t_out(g["dlogits"]), ref["dlogits"])
    errs["dh"] = O.rel_err(as64(g["dh"][:n], dt), ref["dh"]) if n else 0.0
    errs["dx_perm"] = O.rel_err(as64(g["dx_perm"][:n], dt), ref["dx_perm"])
    errs["dx"] = O.rel_err(as64(g["dx"], dt), ref["dx"])
    dw13, dw2 = t_out(g["dw13"]), t_out(g["dw2"])
    off = np.asarray(fwd["offsets"])
    for i in range(wl.E_loc):
        if off[i + 1] == off[i]:
            assert not dw13[i].any() and not dw2[i].any()      # no rows: zero gradients
            continue
        errs[f"dW1[{i}]"] = O.rel_err(dw13[i, :f].T, ref["dW1"][i])
        errs[f"dW3[{i}]"] = O.rel_err(dw13[i, f:].T, ref["dW3"][i])
        errs[f"dW2[{i}]"] = O.rel_err(dw2[i].T, ref["dW2"][i])
    if wg64 is not None:
        errs["dW_g"] = O.rel_err(t_out(g["dw_gate"]), ref["dW_g"])
    worst = max(errs, key=errs.get)
    log(f"{wl.name} T={wl.T} d={wl.d} f={wl.f} E={wl.E} k={wl.k} n={n}: worst {worst} {errs[worst]:.2e}")
    for key, e in errs.items():
        assert e <= tol, (key, e)
    return ref


def test_tiny_fp32():
    wl = make("tiny_fp32")
    w13, w2p, w13_t, w2_t, host = upload(wl, keep_host=True)
    g = train_step(wl, (w13, w2p, w13_t, w2_t), -1)
    check_against_oracle(wl, g, 1e-5, host)


@pytest.mark.parametrize("kw", [
    # capacity drops, remote experts, ragged segments
    dict(T=300, d=256, f=384, E=8, k=2, capacity_factor=0.9, e_begin=2, e_end=7, seed=1),
    # sigmoid gates, k = 4, an expert with no rows
    dict(T=130, d=128, f=192, E=16, k=4, gate="sigmoid_topk_norm", e_begin=0, e_end=16,
         logit_bias="zipf", zipf_beta=3.0, seed=2),
    # many rows per expert: 256-row tiles and remainders in every GEMM
    dict(T=1100, d=512, f=512, E=4, k=2, seed=3),
    # the router in the graph: dx gains the router term, and dW_g
    dict(T=200, d=256, f=256, E=8, k=2, logits_from_gate=True, gate_std=0.05, seed=4),
])
def test_bf16_training_step(kw):
    kw = dict(kw)
    wl = custom("bwd", dtype="bf16", **kw)
    w13, w2p, w13_t, w2_t, host = upload(wl, keep_host=True)
    g = train_step(wl, (w13, w2p, w13_t, w2_t), capacity_of(wl))
    check_against_oracle(wl, g, 1e-2, host)


def test_fp32_with_drops_and_sigmoid():
    wl = custom("bwd32", T=90, d=64, f=128, E=6, k=2, dtype="f32", capacity_factor=0.8,
                e_begin=1, e_end=5, seed=5)
    w13, w2p, w13_t, w2_t, host = upload(wl, keep_host=True)
    g = train_step(wl, (w13, w2p, w13_t, w2_t), capacity_of(wl))
    check_against_oracle(wl, g, 1e-5, host)
    wl = custom("bwd32s", T=70, d=64, f=64, E=8, k=3, dtype="f32", gate="sigmoid_topk_norm",
                seed=6)
    w13, w2p, w13_t, w2_t, host = upload(wl, keep_host=True)
    g = train_step(wl, (w13, w2p, w13_t, w2_t), -1)
    check_against_oracle(wl, g, 1e-5, host)


def test_repeatable_bits():
    """Two backward passes over the same inputs give identical bits (no atomics)."""
    wl = custom("rep", T=257, d=256, f=256, E=8, k=2, capacity_factor=1.0, seed=7)
    ops = upload(wl)[:4]
    C = capacity_of(wl)
    a = train_step(wl, ops, C)
    b = train_step(wl, ops, C)
    n = int(t_out(a["plan"].offsets)[-1])
    for key in ("do_perm", "dh", "dab", "dx_perm"):        # rows past n are never written
        assert np.array_equal(t_out(a[key])[:n], t_out(b[key])[:n]), key
    for key in ("dgate", "dlogits", "dx", "dw13", "dw2"):
        assert np.array_equal(t_out(a[key]), t_out(b[key])), key


def test_mixtral_prefill_training_sampled():
    """The Mixtral-shaped prefill layer (T=4096, d=4096, f=14336, E=8, k=2, router
    in the graph) at full size, as the benchmark runs it: sampled tokens' gate
    gradients and dx, and sampled columns of three experts' weight gradients,
    each computed by the oracle from its definition."""
    wl = make("mixtral_prefill")
    ops = upload(wl, chunk=2)[:4]
    g = train_step(wl, ops, -1)
    k, f, d = wl.k, wl.f, wl.d
    logits = t_out(g["logits"])
    idx, w = O.route(logits, k, wl.gate)
    assert np.array_equal(t_out(g["idx"]), idx)
    plan = O.dispatch(idx, wl.E, -1, 0, wl.E)
    assert np.array_equal(t_out(g["plan"].pair_pos)[:wl.T * k], plan["pair_pos"])
    x64 = O.widen(wl.x, "bf16")
    dy64 = O.widen(output_grad(wl), "bf16")
    wg64 = O.widen(wl.w_gate, "f32")
    cache = {}

    def W(e):
        if e not in cache:
            cache[e] = tuple(O.widen(a, "bf16") for a in wl.expert_weights(e))
        return cache[e]

    tokens = (0, 1234, 4095)
    dgate_ref = np.zeros((len(tokens), k))
    dx_ref = np.zeros((len(tokens), d))
    for i, t in enumerate(tokens):
        for j in range(k):
            w1, w3, w2 = W(int(idx[t, j]))
            dgate_ref[i, j] = float(dy64[t] @ O.swiglu_ffn(x64[t:t + 1], w1, w3, w2)[0])
            eb = B.expert_ffn_backward(x64[t:t + 1], np.array([0, 1]), lambda _: (w1, w3, w2),
                                       w[t, j] * dy64[t:t + 1])
            dx_ref[i] += eb["dx_perm"][0]
        dl = B.gate_backward(logits[t:t + 1], idx[t:t + 1], dgate_ref[i:i + 1], wl.gate)
        dx_ref[i] += (dl @ wg64.T)[0]
    sel = list(tokens)
    e_dg = O.rel_err(t_out(g["dgate"])[sel], dgate_ref)
    e_dx = O.rel_err(as64(g["dx"], "bf16")[sel], dx_ref)
    log(f"mixtral training: sampled dgate err {e_dg:.2e}, dx err {e_dx:.2e}")
    assert e_dg <= 1e-2 and e_dx <= 1e-2
    # weight-gradient columns: the FFN splits over the f columns, so the oracle's
    # backward of the sub-FFN on columns S gives exactly dW1[:, S], dW3[:, S], dW2[S, :]
    off, sp = plan["offsets"], plan["sorted_pair"]
    dw13, dw2 = g["dw13"], g["dw2"]
    S = np.array([0, 777, 14335])
    for e in (0, 3, 7):
        r0, r1 = int(off[e]), int(off[e + 1])
        pairs = sp[r0:r1].astype(np.int64)
        toks, js = pairs // k, pairs % k
        do_e = w[toks, js][:, None] * dy64[toks]
        w1, w3, w2 = W(e)
        eb = B.expert_ffn_backward(x64[toks], np.array([0, r1 - r0]),
                                   lambda _: (w1[:, S], w3[:, S], w2[S, :]), do_e)
        got1 = dw13[e, torch.from_numpy(S).to(DEV)].cpu().numpy()
        got3 = dw13[e, torch.from_numpy(S + f).to(DEV)].cpu().numpy()
        got2 = dw2[e][:, torch.from_numpy(S).to(DEV)].cpu().numpy()
        errs = (O.rel_err(got1, eb["dW1"][0].T), O.rel_err(got3, eb["dW3"][0].T),
                O.rel_err(got2, eb["dW2"][0].T))
        log(f"mixtral training: expert {e} ({r1 - r0} rows) dW1/dW3/dW2 column errs "
            + " ".join(f"{v:.2e}" for v in errs))
        assert max(errs) <= 1e-2


@pytest.mark.parametrize("kw", [
    dict(T=50, d=128, f=128, E=4, k=2, capacity_factor=0.0, seed=8),      # capacity 0: every pair drops
    dict(T=40, d=128, f=192, E=4, k=4, seed=9),                           # k = E
    dict(T=1, d=64, f=64, E=8, k=2, seed=10),                              # one token, most experts empty
    dict(T=64, d=128, f=128, E=8, k=2, e_begin=3, e_end=4, seed=11),      # one local expert
])
def test_backward_edge_cases(kw):
    wl = custom("edge", dtype="bf16", **kw)
    w13, w2p, w13_t, w2_t, host = upload(wl, keep_host=True)
    C = capacity_of(wl)
    g = train_step(wl, (w13, w2p, w13_t, w2_t), C)
    n = int(t_out(g["plan"].offsets)[-1])
    if C == 0:
        assert n == 0
        assert not t_out(g["dx"]).any() and not t_out(g["dgate"]).any()
        assert not t_out(g["dlogits"]).any()
        assert not t_out(g["dw13"]).any() and not t_out(g["dw2"]).any()
    check_against_oracle(wl, g, 1e-2, host)
