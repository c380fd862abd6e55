"""Pins of the NSA backward oracle (CPU only): finite differences, the closed
form of the gate gradient, the window-only case against a library attention
backward, and the structure the pages fix (top-n is a no-op on the graph)."""
from dataclasses import dataclass

import numpy as np
import pytest
import torch

from oracle import nsa_backward as NB
from oracle import nsa_oracle as O


@dataclass(frozen=True)
class P:
    l: int = 4
    d: int = 2
    l_sel: int = 4
    n_sel: int = 2
    n_local: int = 1
    force_initial: int = 1
    w: int = 3


def _case(seed, T=12, G=2, dk=4, dv=3, p=P()):
    rng = np.random.default_rng(seed)
    return dict(Q=rng.standard_normal((T, G, dk)), K=rng.standard_normal((T, dk)), V=rng.standard_normal((T, dv)),
                Wk=rng.standard_normal((p.l * dk, dk)) / 4, PEk=rng.standard_normal((p.l, dk)) * 0.1,
                Wv=rng.standard_normal((p.l * dv, dv)) / 4, PEv=rng.standard_normal((p.l, dv)) * 0.1,
                gates=rng.uniform(0.1, 0.9, (T, G, 3)), dout=rng.standard_normal((T, G, dv)))


def test_gradients_match_finite_differences():
    """Autograd's derivative of the restated forward against central differences
    (torch.autograd.gradcheck, float64), every input at once."""
    c = _case(0)
    p = P()
    rows = [3, 7, 11]
    sel = NB.sequence_backward(**c, rows=rows, p=p)["sel"]
    names = ["Q", "K", "V", "Wk", "PEk", "Wv", "PEv", "gates"]
    tens = [torch.tensor(c[n], dtype=torch.float64, requires_grad=True) for n in names]
    dout = torch.tensor(c["dout"], dtype=torch.float64)

    def f(Q, K, V, Wk, PEk, Wv, PEv, gates):
        Kc = NB.compress_t(K, Wk, PEk, p.l, p.d)
        Vc = NB.compress_t(V, Wv, PEv, p.l, p.d)
        tot = torch.zeros((), dtype=torch.float64)
        for r, t in enumerate(rows):
            tot = tot + (NB.query_out_t(Q[t], K, V, Kc, Vc, t, gates[t], p, sel[r], 0.5) * dout[t]).sum()
        return tot

    assert torch.autograd.gradcheck(f, tens, eps=1e-6, atol=1e-7, rtol=1e-5)


def test_gate_gradient_closed_form():
    """d loss / d g_br[t, h] = dout[t, h] . o_br[t, h] (the output is linear in the gates)."""
    c = _case(1)
    p = P()
    rows = [5, 9]
    g = NB.sequence_backward(**c, rows=rows, p=p)
    Kc = O.compress(c["K"], c["Wk"], c["PEk"], p.l, p.d)
    Vc = O.compress(c["V"], c["Wv"], c["PEv"], p.l, p.d)
    for r, t in enumerate(rows):
        res = O.nsa_query(c["Q"][t], c["K"], c["V"], Kc, Vc, t, c["gates"][t], p.l, p.d, p.l_sel, p.n_sel,
                          p.n_local, p.force_initial, p.w, override_idx=g["sel"][r])
        want = np.stack([(c["dout"][t] * o).sum(axis=1) for o in (res.o_cmp, res.o_slc, res.o_win)], axis=1)
        # both oracles use the bf16-rounded compressed cache, so the branch outputs agree exactly
        np.testing.assert_allclose(g["dgates"][t], want, rtol=1e-12, atol=1e-12)
    assert np.all(g["dgates"][[t for t in range(12) if t not in rows]] == 0.0)


def test_window_only_equals_library_attention_backward():
    """Gates (0, 0, 1): the gradients are those of sliding-window causal attention,
    here taken from torch's scaled_dot_product_attention in float64."""
    c = _case(2, T=10)
    p = P()
    c["gates"] = np.zeros_like(c["gates"])
    c["gates"][..., 2] = 1.0
    rows = list(range(10))
    g = NB.sequence_backward(**c, rows=rows, p=p)
    T, G, dk = c["Q"].shape
    q = torch.tensor(c["Q"].transpose(1, 0, 2), dtype=torch.float64, requires_grad=True)     # [G, T, dk]
    k = torch.tensor(np.broadcast_to(c["K"], (G,) + c["K"].shape).copy(), dtype=torch.float64, requires_grad=True)
    v = torch.tensor(np.broadcast_to(c["V"], (G,) + c["V"].shape).copy(), dtype=torch.float64, requires_grad=True)
    i = torch.arange(T)[:, None]
    j = torch.arange(T)[None, :]
    mask = (j <= i) & (i - j < p.w)
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask)
    (o * torch.tensor(c["dout"].transpose(1, 0, 2))).sum().backward()
    np.testing.assert_allclose(g["dQ"], q.grad.numpy().transpose(1, 0, 2), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(g["dK"], k.grad.sum(0).numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(g["dV"], v.grad.sum(0).numpy(), rtol=1e-10, atol=1e-12)
    for n in ("dWk", "dPEk", "dWv", "dPEv"):
        assert np.all(g[n] == 0.0)


def test_top_n_is_a_no_op_on_the_graph():
    """Selected-branch gates only: the selection was made from the compressed branch's
    scores, yet the compression weights receive exactly zero gradient, and so do the
    tokens of unselected blocks.  Compressed-branch gates only: the trailing incomplete
    block receives none (it is in no visible compressed block)."""
    p = P(l=4, d=2, l_sel=4, n_sel=3, n_local=1, force_initial=1, w=2)
    c = _case(3, T=24, p=p)
    c["gates"] = np.zeros_like(c["gates"])
    c["gates"][..., 1] = 1.0
    g = NB.sequence_backward(**c, rows=[23], p=p)
    sel = g["sel"][0]
    assert len(sel) == 3 and 0 in sel and 5 in sel         # forced initial and local blocks, one routed
    for n in ("dWk", "dPEk", "dWv", "dPEv"):
        assert np.all(g[n] == 0.0)
    unsel = [x for x in range(24) if x // p.l_sel not in sel]
    assert np.all(g["dK"][unsel] == 0.0) and np.all(g["dV"][unsel] == 0.0)
    assert np.any(g["dK"][[x for x in range(24) if x // p.l_sel in sel]] != 0.0)
    c["gates"] = np.zeros_like(c["gates"])
    c["gates"][..., 0] = 1.0
    g = NB.sequence_backward(**c, rows=[12], p=p)               # blocks 0..4 cover tokens 0..11
    assert np.all(g["dK"][12:] == 0.0) and np.all(g["dV"][12:] == 0.0)
    assert np.any(g["dK"][:12] != 0.0) and np.any(g["dWk"] != 0.0)


def test_gate_network_gradients_match_finite_differences():
    """With the gate network, autograd's derivatives with respect to the queries
    (both paths), the gate weights and the bias against central differences."""
    c = _case(4)
    p = P()
    rows = [2, 6, 11]
    rng = np.random.default_rng(5)
    Wg = rng.standard_normal((2, 3, 4)) * 0.5
    bg = rng.standard_normal((2, 3)) * 0.5
    sel = NB.sequence_backward(**c, rows=rows, p=p)["sel"]
    tens = [torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (c["Q"], Wg, bg)]
    K, V = (torch.tensor(c[n], dtype=torch.float64) for n in ("K", "V"))
    Kc = NB.compress_t(K, torch.tensor(c["Wk"]), torch.tensor(c["PEk"]), p.l, p.d)
    Vc = NB.compress_t(V, torch.tensor(c["Wv"]), torch.tensor(c["PEv"]), p.l, p.d)
    dout = torch.tensor(c["dout"], dtype=torch.float64)

    def f(Q, W, b):
        tot = torch.zeros((), dtype=torch.float64)
        for r, t in enumerate(rows):
            gts = torch.sigmoid(torch.einsum("hck,hk->hc", W, Q[t]) + b)
            tot = tot + (NB.query_out_t(Q[t], K, V, Kc, Vc, t, gts, p, sel[r], 0.5) * dout[t]).sum()
        return tot

    assert torch.autograd.gradcheck(f, tens, eps=1e-6, atol=1e-7, rtol=1e-5)
    # and sequence_backward with the gate network returns those same derivatives
    r = NB.sequence_backward(**c, rows=rows, p=p, sel=sel, scale=0.5, round_cmp=False, Wg=Wg, bg=bg)
    for x in tens:
        x.grad = None
    f(*tens).backward()
    np.testing.assert_allclose(r["dQ"], tens[0].grad.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(r["dWg"], tens[1].grad.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(r["dbg"], tens[2].grad.numpy(), rtol=1e-12, atol=1e-12)
