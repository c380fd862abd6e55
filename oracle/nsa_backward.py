"""Float64 backward oracle of the NSA forward pass (gradients for training).

TEST INFRASTRUCTURE ONLY.  Only the test suite may import this module; the
library never does.  It shares no code with the HIP path.

Sources: [LES] lesson "Native Sparse Attention (DeepSeek NSA)", AI Engineering
from Scratch, phase 10 · 17 (Hindi), section on why NSA is natively trainable:
the top-k selection only decides which blocks are loaded and is a no-op on the
graph of the forward computation; gradients flow through the compressed branch
(its output, hence the compressed keys and values and the compression MLP) and
through the selected and window branches.  [FLI] lesson 5.5/02, section
"NSA: три ветви": the output equation and the three branches.

The forward of nsa_oracle.nsa_query is restated with float64 torch tensors so
that autograd takes the derivative of the scalar  sum_{t,h} dout[t,h] . out[t,h].
The selected block ids are constants (from the forward oracle's top-n).  The
forward stores the compressed cache in bf16, so by default the values used here
are the rounded ones (exactly the forward oracle's), while the derivative of the
rounding is taken as the identity (it is zero almost everywhere, and a rounding
step passes the gradient through unchanged).
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np
import torch

from oracle import nsa_oracle as O

F64 = torch.float64


def compress_t(K: torch.Tensor, W: torch.Tensor, PE: torch.Tensor, l: int, d: int,
               round_bf16: bool = False) -> torch.Tensor:
    """Compressed keys (or values) of one sequence and head: (K[i*d : i*d+l] + PE) flattened, times W.

    With round_bf16 the value is rounded to bf16 as the forward stores it; the
    gradient passes through the rounding unchanged."""
    nc = O.n_compressed(K.shape[0], l, d)
    if nc == 0:
        return torch.zeros((0, W.shape[1]), dtype=F64)
    X = torch.stack([(K[i * d:i * d + l] + PE).reshape(-1) for i in range(nc)])
    Y = X @ W
    if round_bf16:
        Y = Y + (torch.from_numpy(O.round_to_bf16(Y.detach().numpy())) - Y).detach()
    return Y


def attend_t(q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, scale: float) -> torch.Tensor:
    """Softmax attention of q [H, dk] over K [n, dk], V [n, dv]; zero output when n == 0."""
    if K.shape[0] == 0:
        return torch.zeros((q.shape[0], V.shape[1]), dtype=F64)
    p = torch.softmax(scale * (q @ K.T), dim=1)
    return p @ V


def query_out_t(q, K, V, Kc, Vc, t: int, gates, p, idx: Sequence[int], scale: float):
    """Differentiable NSA output of one position's group heads, given the selected ids."""
    nvis = O.n_compressed(t + 1, p.l, p.d)
    o_cmp = attend_t(q, Kc[:nvis], Vc[:nvis], scale)
    toks = np.concatenate([np.arange(j * p.l_sel, min((j + 1) * p.l_sel, t + 1)) for j in idx])
    o_slc = attend_t(q, K[toks], V[toks], scale)
    wt = np.arange(max(0, t - p.w + 1), t + 1)
    o_win = attend_t(q, K[wt], V[wt], scale)
    return gates[:, 0:1] * o_cmp + gates[:, 1:2] * o_slc + gates[:, 2:3] * o_win


def sequence_backward(Q: np.ndarray, K: np.ndarray, V: np.ndarray, Wk: np.ndarray, PEk: np.ndarray,
                      Wv: np.ndarray, PEv: np.ndarray, gates: np.ndarray, dout: np.ndarray, rows: Sequence[int],
                      p, sel: Optional[Sequence[Sequence[int]]] = None, scale: Optional[float] = None,
                      round_cmp: bool = True, Wg: Optional[np.ndarray] = None,
                      bg: Optional[np.ndarray] = None) -> dict:
    """Gradients of  sum_{t in rows} sum_h dout[t,h] . out[t,h]  for one sequence and KV group.

    Q [T, G, dk] (the group's query heads per position), K [T, dk], V [T, dv], Wk [l*dk, dk],
    PEk [l, dk], Wv [l*dv, dv], PEv [l, dv], gates [T, G, 3], dout [T, G, dv].
    ``sel`` gives the selected block ids per row; by default the forward oracle's top-n.
    ``round_cmp`` uses the bf16-rounded compressed cache values (as the forward does).
    With ``Wg`` [G, 3, dk] (and optionally ``bg`` [G, 3]) the gates come from the gate
    network, gate[t, h, c] = sigmoid(Wg[h, c] . Q[t, h] + bg[h, c]) (``gates`` is then
    ignored), and dWg, dbg are returned too; dQ then includes the gates' path.
    Returns float64 numpy arrays: dQ, dK, dV, dWk, dPEk, dWv, dPEv, dgates (shapes of the inputs; dgates
    is the gradient reaching the gate values), and dKc, dVc: the gradients reaching the compressed
    cache [nc, dk] / [nc, dv]; with the gate network also dWg and dbg.
    """
    dk_ = Q.shape[2]
    s = 1.0 / np.sqrt(dk_) if scale is None else scale
    Qt = torch.tensor(Q, dtype=F64, requires_grad=True)
    Kt = torch.tensor(K, dtype=F64, requires_grad=True)
    Vt = torch.tensor(V, dtype=F64, requires_grad=True)
    Wkt = torch.tensor(Wk, dtype=F64, requires_grad=True)
    PEkt = torch.tensor(PEk, dtype=F64, requires_grad=True)
    Wvt = torch.tensor(Wv, dtype=F64, requires_grad=True)
    PEvt = torch.tensor(PEv, dtype=F64, requires_grad=True)
    Gt = torch.tensor(gates, dtype=F64, requires_grad=True)
    Wgt = bgt = None
    if Wg is not None:
        Wgt = torch.tensor(Wg, dtype=F64, requires_grad=True)
        z = torch.einsum("hck,thk->thc", Wgt, Qt)
        if bg is not None:
            bgt = torch.tensor(bg, dtype=F64, requires_grad=True)
            z = z + bgt
        gate_vals = torch.sigmoid(z)
        gate_vals.retain_grad()  # dgates: the gradient reaching the gate values, dout . o per branch
    else:
        gate_vals = Gt
    Kc = compress_t(Kt, Wkt, PEkt, p.l, p.d, round_cmp)
    Vc = compress_t(Vt, Wvt, PEvt, p.l, p.d, round_cmp)
    for c in (Kc, Vc):
        if c.requires_grad:
            c.retain_grad()
    if sel is None:  # the forward oracle's selection (with the bf16-rounded compressed cache)
        Kc_o = O.compress(K, Wk, PEk, p.l, p.d)
        Vc_o = O.compress(V, Wv, PEv, p.l, p.d)
        sel = [O.nsa_query(Q[t], K, V, Kc_o, Vc_o, int(t), gates[t], p.l, p.d, p.l_sel, p.n_sel, p.n_local,
                           p.force_initial, p.w, scale=s).idx for t in rows]
    loss = torch.zeros((), dtype=F64)
    for r, t in enumerate(rows):
        out = query_out_t(Qt[t], Kt, Vt, Kc, Vc, int(t), gate_vals[t], p, sel[r], s)
        loss = loss + (out * torch.tensor(dout[t], dtype=F64)).sum()
    loss.backward()
    g = lambda x: (x.grad if x.grad is not None else torch.zeros_like(x)).detach().numpy()
    res = dict(dQ=g(Qt), dK=g(Kt), dV=g(Vt), dWk=g(Wkt), dPEk=g(PEkt), dWv=g(Wvt), dPEv=g(PEvt), dgates=g(Gt),
               dKc=g(Kc), dVc=g(Vc), sel=sel)
    if Wgt is not None:
        res["dgates"] = g(gate_vals)
        res["dWg"] = g(Wgt)
        res["dbg"] = g(bgt) if bgt is not None else None
    return res
