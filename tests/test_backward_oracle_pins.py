"""Pins of the backward oracle against what fixes it from outside:

  * central finite differences of L = <dout, out> (the forward oracle) with respect to
    every input and weight, on small inputs whose routing has clear margins (the
    selection is piecewise constant, so the perturbation must not flip it);
  * torch's fp64 autograd of an independent, per-token formulation of the layer
    (no permutation, no padding: each token through its experts directly).
"""
import numpy as np
import pytest
import torch

from oracle import moe_backward_oracle as BW
from oracle import moe_oracle as O


def _problem(seed, T=6, d=8, E=4, k=2, d_e=6, shared=True, routed=False):
    rng = np.random.default_rng(seed)
    p = dict(
        x=rng.standard_normal((T, d)),
        w1=rng.standard_normal((E, d, d_e)) / np.sqrt(d),
        w3=rng.standard_normal((E, d, d_e)) / np.sqrt(d),
        w2=rng.standard_normal((E, d_e, d)) / np.sqrt(d_e),
        w_gate=rng.standard_normal((d, E)) / np.sqrt(d),
        bias=rng.standard_normal(E) * 0.5,
        dout=rng.standard_normal((T, d)),
    )
    if shared:
        p.update(ws1=rng.standard_normal((d, d_e)) / np.sqrt(d),
                 ws3=rng.standard_normal((d, d_e)) / np.sqrt(d),
                 ws2=rng.standard_normal((d_e, d)) / np.sqrt(d_e))
    if routed:
        p["topk_idx"] = rng.integers(0, E, size=(T, k))          # duplicates allowed
        p["topk_w"] = rng.random((T, k))
    return p


def _forward(p, k, block_m, renormalize, routed):
    """The forward definition with the routing weights taken from the fp64 logits (the
    forward oracle takes them from the fp32-rounded logits the device keeps, a step
    function at the scale of a finite-difference step), the selection from fp32."""
    kw = dict(k=k, block_m=block_m, ws1=p.get("ws1"), ws3=p.get("ws3"), ws2=p.get("ws2"))
    if routed:
        return O.moe_layer(p["x"], p["w1"], p["w3"], p["w2"], topk_idx=p["topk_idx"],
                           topk_w=p["topk_w"], **kw)
    logits = O.router_logits(p["x"], p["w_gate"], p["bias"])
    idx = O.topk_by_repeated_max(logits.astype(np.float32), k)
    w = O.gate_weights(logits, idx, renormalize)
    fwd = O.moe_layer(p["x"], p["w1"], p["w3"], p["w2"], topk_idx=idx, topk_w=w, **kw)
    fwd.logits = logits
    return fwd


def _grads(p, k, block_m, renormalize, routed):
    fwd = _forward(p, k, block_m, renormalize, routed)
    return fwd, BW.moe_layer_backward(fwd, p["x"], p["w1"], p["w3"], p["w2"], p["dout"], k=k,
                                      block_m=block_m, w_gate=p["w_gate"], bias=p["bias"],
                                      renormalize=renormalize, ws1=p.get("ws1"),
                                      ws3=p.get("ws3"), ws2=p.get("ws2"), routed=routed)


@pytest.mark.parametrize("renormalize,routed,shared", [(False, False, True), (True, False, False),
                                                       (False, True, True)])
def test_finite_differences(renormalize, routed, shared):
    k, block_m, h = 2, 4, 1e-6
    p = _problem(7 + renormalize + 2 * routed, shared=shared, routed=routed)
    fwd, g = _grads(p, k, block_m, renormalize, routed)
    loss = lambda q: float(np.sum(q["dout"] * _forward(q, k, block_m, renormalize, routed).out))
    names = ["x", "w1", "w3", "w2"] + (["ws1", "ws3", "ws2"] if shared else [])
    names += [] if routed else ["w_gate", "bias"]
    grad_of = {"x": g.dx, "w1": g.dw1, "w3": g.dw3, "w2": g.dw2, "ws1": g.dws1, "ws3": g.dws3,
               "ws2": g.dws2, "w_gate": g.dw_gate, "bias": g.dbias}
    checked = 0
    for n in names:
        flat = p[n].reshape(-1)
        for i in range(flat.size):
            q_plus = {kk: (v.copy() if isinstance(v, np.ndarray) else v) for kk, v in p.items()}
            q_minus = {kk: (v.copy() if isinstance(v, np.ndarray) else v) for kk, v in p.items()}
            q_plus[n].reshape(-1)[i] += h
            q_minus[n].reshape(-1)[i] -= h
            if not routed:
                sel = lambda q: _forward(q, k, block_m, renormalize, routed).topk_idx
                if not (np.array_equal(sel(q_plus), fwd.topk_idx) and
                        np.array_equal(sel(q_minus), fwd.topk_idx)):
                    continue
            num = (loss(q_plus) - loss(q_minus)) / (2 * h)
            ana = grad_of[n].reshape(-1)[i]
            assert abs(num - ana) <= 1e-6 * max(1.0, abs(ana)), (n, i, num, ana)
            checked += 1
    assert checked > 200


def _torch_layer(p, k, renormalize, routed):
    t = {n: torch.tensor(v, dtype=torch.float64, requires_grad=True)
         for n, v in p.items() if n not in ("topk_idx", "topk_w", "dout")}
    x = t["x"]
    T = x.shape[0]
    if routed:
        idx = torch.tensor(p["topk_idx"])
        w = torch.tensor(p["topk_w"], dtype=torch.float64)
    else:
        logits = x @ t["w_gate"] + t["bias"]
        prob = torch.softmax(logits, dim=1)
        idx = torch.tensor(O.topk_by_repeated_max(logits.detach().numpy(), k))
        w = torch.gather(prob, 1, idx)
        if renormalize:
            w = w / w.sum(dim=1, keepdim=True)
    rows = []
    for i in range(T):
        acc = torch.zeros(x.shape[1], dtype=torch.float64)
        for j in range(k):
            e = int(idx[i, j])
            h = torch.nn.functional.silu(x[i] @ t["w1"][e]) * (x[i] @ t["w3"][e])
            acc = acc + w[i, j] * (h @ t["w2"][e])
        if "ws1" in t:
            h = torch.nn.functional.silu(x[i] @ t["ws1"]) * (x[i] @ t["ws3"])
            acc = acc + h @ t["ws2"]
        rows.append(acc)
    out = torch.stack(rows)
    (out * torch.tensor(p["dout"])).sum().backward()
    return {n: v.grad.numpy() for n, v in t.items() if v.grad is not None}


@pytest.mark.parametrize("renormalize,routed", [(False, False), (True, False), (False, True)])
def test_matches_torch_autograd_of_a_per_token_formulation(renormalize, routed):
    k, block_m = 3, 8
    p = _problem(11 + renormalize, T=20, d=16, E=6, k=k, d_e=12, shared=True, routed=routed)
    _, g = _grads(p, k, block_m, renormalize, routed)
    ref = _torch_layer(p, k, renormalize, routed)
    ours = {"x": g.dx, "w1": g.dw1, "w3": g.dw3, "w2": g.dw2, "ws1": g.dws1, "ws3": g.dws3,
            "ws2": g.dws2}
    if not routed:
        ours.update(w_gate=g.dw_gate, bias=g.dbias)
    for n, v in ours.items():
        np.testing.assert_allclose(v, ref[n], rtol=1e-10, atol=1e-12, err_msg=n)


def test_experts_without_rows_get_zero_weight_gradients():
    p = _problem(3, routed=True, shared=False)
    p["topk_idx"][:] = 1                                   # only expert 1 has rows
    _, g = _grads(p, 2, 4, False, True)
    for e in (0, 2, 3):
        assert not g.dw1[e].any() and not g.dw3[e].any() and not g.dw2[e].any()
    assert g.dw1[1].any()
