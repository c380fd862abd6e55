"""GPU parity of the NSA backward (nsa_prefill_bwd + nsa_compress_bwd) against
the float64 autograd oracle of oracle/nsa_backward.py.

Tolerance: the kernels round the probabilities P and dS = P (dP - D) to bf16 as
MFMA operands (relative error 2^-9 each) and sum in fp32.  Every gradient is a
sum of such products over up to a few thousand keys or queries, so the error
of a sum is a small multiple of 2^-9 times the size of its terms, and the sums
partly cancel.  Each tensor is compared as a whole: max |gpu - oracle| <=
3e-2 * max |oracle| and mean |gpu - oracle| <= 3e-3 * max |oracle|.  The
compressed-cache gradients pass through a second product (dX = dY W^T, fp32)
and the same bound applies.
"""
import numpy as np
import pytest
import torch

import long_context_sparse_nsa_amd as N
import nsa_inputs as I
from oracle import nsa_backward as NB
from oracle import nsa_oracle as O
from tests import gpu_util as U

pytestmark = pytest.mark.gpu

MAX_REL = 3e-2
MEAN_REL = 3e-3


def _w(bits):
    return U.bits_to_f64(np.asarray(bits))


def close(got, want, what, scale=None):
    """Whole-tensor comparison; `scale` (default max |want|) is the size the errors are measured against."""
    got, want = np.asarray(got, dtype=np.float64), np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    scale = max(float(np.abs(want).max()) if scale is None else float(scale), 1e-30)
    err = np.abs(got - want)
    print(f"{what}: max {err.max() / scale:.2e} mean {err.mean() / scale:.2e} (scale {scale:.3e})")
    assert err.max() <= MAX_REL * scale, f"{what}: max-abs error {err.max():.3e} > {MAX_REL} x {scale:.3e}"
    assert err.mean() <= MEAN_REL * scale, f"{what}: mean-abs error {err.mean():.3e} > {MEAN_REL} x {scale:.3e}"


def oracle_cache(case):
    """The oracle's bf16-rounded compressed cache of every (b, g): bits [B, H, nc, D]."""
    wl = case.wl
    kc, vc = [], []
    for b in range(wl.batch):
        kb, vb = [], []
        for g in range(wl.num_kv_heads):
            _, _, Kc, Vc = O.compress_group(case, b, g)
            kb.append(U.f64_to_bits(Kc))
            vb.append(U.f64_to_bits(Vc))
        kc.append(np.stack(kb))
        vc.append(np.stack(vb))
    return np.stack(kc), np.stack(vc)


def run_backward(case, dout_bits, saved_lse=True):
    """GPU forward (for the selection and, with saved_lse, each branch's log-sum-exp)
    and backward with the oracle's compressed cache."""
    wl, p = case.wl, case.p
    dims, cfg = U.dims_cfg(case)
    B, Hq, H, dk, dv, T = wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.d_k, wl.d_v, wl.seq_len
    nc = N.compressed_count(T, p.l, p.d)
    kc_bits, vc_bits = oracle_cache(case) if nc > 0 else (None, None)
    if nc > 0:
        _, sel, lse = U.run_prefill(case, kc_bits=kc_bits, vc_bits=vc_bits, with_lse=True)
    else:
        _, sel, lse = U.run_prefill(case, with_lse=True)
    lse_t = torch.from_numpy(np.ascontiguousarray(lse, dtype=np.float32)).cuda() if saved_lse else None
    nanf = lambda *s: torch.full(s, float("nan"), dtype=torch.float32, device="cuda")
    q, k, v = U.dev_bits(case.q), U.dev_bits(case.k), U.dev_bits(case.v)
    kc = U.dev_bits(kc_bits) if nc > 0 else None
    vc = U.dev_bits(vc_bits) if nc > 0 else None
    gates, wg, bgt = U.gate_args(case)
    sel_t = torch.from_numpy(np.ascontiguousarray(sel, dtype=np.int32)).cuda()
    dq, dK, dV, dgates = nanf(B, T, Hq, dk), nanf(B, H, T, dk), nanf(B, H, T, dv), nanf(B, T, Hq, 3)
    dkc = nanf(B, H, nc, dk) if nc > 0 else None
    dvc = nanf(B, H, nc, dv) if nc > 0 else None
    dwg = nanf(Hq, 3, dk) if wg is not None else None
    dbg = nanf(Hq, 3) if bgt is not None else None
    ws = N.new_workspace(N.nsa_prefill_bwd_workspace_size(dims, cfg, T))
    N.nsa_prefill_bwd(dims, cfg, T, q, k, v, kc, vc, gates, sel_t, U.dev_bits(dout_bits), dq, dK, dV, dkc, dvc,
                      dgates, ws, w_gate=wg, b_gate=bgt, dw_gate=dwg, db_gate=dbg, lse=lse_t)
    dk_raw, dv_raw = dK.clone(), dV.clone()
    res = dict(sel=sel, dq=dq, dk_raw=dk_raw, dv_raw=dv_raw, dkc=dkc, dvc=dvc, dgates=dgates, dwg=dwg, dbg=dbg)
    for which, x, w_bits, pe_bits, dy, dx, D in ((0, k, case.w_k, case.pe_k, dkc, dK, dk),
                                                 (1, v, case.w_v, case.pe_v, dvc, dV, dv)):
        dw, dpe = nanf(p.l * D, D), nanf(p.l, D)
        wsc = N.new_workspace(N.nsa_compress_bwd_workspace_size(dims, cfg, T, which))
        N.nsa_compress_bwd(dims, cfg, T, which, x, U.dev_bits(w_bits), U.dev_bits(pe_bits), dy, dx, dw, dpe, wsc)
        res["dw" + "kv"[which]] = dw
        res["dpe" + "kv"[which]] = dpe
    res["dk"], res["dv"] = dK, dV
    torch.cuda.synchronize()
    return {n: (t.cpu().numpy() if isinstance(t, torch.Tensor) else t) for n, t in res.items()}


def oracle_group(case, dout_bits, sel, b, g, rows):
    wl, p = case.wl, case.p
    G = wl.num_q_heads // wl.num_kv_heads
    hs = slice(g * G, (g + 1) * G)
    sl = [[int(j) for j in sel[b, t, g] if j >= 0] for t in rows]
    net = getattr(case, "gate_net", False)
    Wg = _w(case.w_gate[hs]) if net else None
    bg = np.asarray(case.b_gate[hs], dtype=np.float64) if net and case.b_gate is not None else None
    return NB.sequence_backward(_w(case.q[b, :, hs]), _w(case.k[b, g]), _w(case.v[b, g]), _w(case.w_k),
                                _w(case.pe_k), _w(case.w_v), _w(case.pe_v),
                                np.asarray(case.gates[b, :, hs], dtype=np.float64), _w(dout_bits[b, :, hs]),
                                list(rows), p, sel=sl, Wg=Wg, bg=bg)


def oracle_rows(case, dout_bits, sel, b, g, rows):
    """dq and dgates of single positions: the oracle's per-position output
    (NB.query_out_t) differentiated with respect to that position's query heads
    and gates, the caches held constant (one position's terms do not involve the
    others)."""
    wl, p = case.wl, case.p
    G = wl.num_q_heads // wl.num_kv_heads
    hs = slice(g * G, (g + 1) * G)
    K, V, Kc, Vc = (torch.from_numpy(np.asarray(x, dtype=np.float64)) for x in O.compress_group(case, b, g))
    scale = 1.0 / np.sqrt(wl.d_k)
    out = {}
    for t in rows:
        q = torch.tensor(_w(case.q[b, t, hs]), dtype=torch.float64, requires_grad=True)
        gt = torch.tensor(np.asarray(case.gates[b, t, hs], dtype=np.float64), requires_grad=True)
        idx = [int(j) for j in sel[b, t, g] if j >= 0]
        o = NB.query_out_t(q, K, V, Kc, Vc, int(t), gt, p, idx, scale)
        (o * torch.from_numpy(_w(dout_bits[b, t, hs]))).sum().backward()
        out[t] = (q.grad.numpy(), gt.grad.numpy())
    return out


def check_all(case, dout_bits, got):
    wl = case.wl
    G = wl.num_q_heads // wl.num_kv_heads
    T = wl.seq_len
    acc = {n: [] for n in ("dq", "dgates", "dk", "dv", "dkc", "dvc")}
    want = {n: [] for n in acc}
    sums = {n: 0.0 for n in ("dWk", "dPEk", "dWv", "dPEv")}
    dwg = np.zeros((wl.num_q_heads, 3, wl.d_k))  # gate network: per head, summed over sequences
    dbg = np.zeros((wl.num_q_heads, 3))
    terms = {"k": 0.0, "v": 0.0}  # sum_i |dY_i| over every (b, g): the size of dPE's terms
    for b in range(wl.batch):
        for g in range(wl.num_kv_heads):
            r = oracle_group(case, dout_bits, got["sel"], b, g, range(T))
            hs = slice(g * G, (g + 1) * G)
            pairs = (("dq", got["dq"][b, :, hs], r["dQ"]), ("dgates", got["dgates"][b, :, hs], r["dgates"]),
                     ("dk", got["dk"][b, g], r["dK"]), ("dv", got["dv"][b, g], r["dV"]))
            if got["dkc"] is not None:
                pairs += (("dkc", got["dkc"][b, g], r["dKc"]), ("dvc", got["dvc"][b, g], r["dVc"]))
            for n, a, w in pairs:
                acc[n].append(a)
                want[n].append(w)
            for n in sums:
                sums[n] = sums[n] + r[n]
            terms["k"] = terms["k"] + np.abs(r["dKc"]).sum(axis=0)
            terms["v"] = terms["v"] + np.abs(r["dVc"]).sum(axis=0)
            if "dWg" in r:
                dwg[hs] += r["dWg"]
                if r["dbg"] is not None:
                    dbg[hs] += r["dbg"]
    # A gradient that is exactly 0 (e.g. dq, dk when every branch sees one key, so
    # each dS = P (dP - D) cancels) is measured against the size of the terms that
    # cancel, bounded below by 1e-6 x the dgates scale (dout . o).
    floor = 1e-6 * float(np.abs(np.stack(want["dgates"])).max()) / MAX_REL
    for n in acc:
        if acc[n]:
            w = np.stack(want[n])
            close(np.stack(acc[n]), w, n, scale=max(float(np.abs(w).max()), floor))
    close(got["dwk"], sums["dWk"], "dWk")
    # dPE = (sum_i dY_i) W^T.  For keys sum_i dKc_i is 0 up to rounding (every
    # softmax's dS sums to 0 over its keys), so dPE_k is near 0 and its error is
    # measured against the size of the summed terms, (sum_i |dY_i|) |W|^T.
    wk, wv = np.abs(_w(case.w_k)), np.abs(_w(case.w_v))
    D_k, D_v = wl.d_k, wl.d_v
    size_k = (wk.reshape(-1, D_k) @ np.broadcast_to(terms["k"], (D_k,))).max() if np.ndim(terms["k"]) else 0.0
    size_v = (wv.reshape(-1, D_v) @ np.broadcast_to(terms["v"], (D_v,))).max() if np.ndim(terms["v"]) else 0.0
    close(got["dpek"], sums["dPEk"], "dPEk", scale=max(size_k, float(np.abs(sums["dPEk"]).max())))
    close(got["dwv"], sums["dWv"], "dWv")
    close(got["dpev"], sums["dPEv"], "dPEv", scale=max(size_v, float(np.abs(sums["dPEv"]).max())))
    if got.get("dwg") is not None:
        close(got["dwg"], dwg, "dw_gate")
    if got.get("dbg") is not None:
        close(got["dbg"], dbg, "db_gate")


def test_backward_tiny_all_rows():
    case = I.generate(I.workload("tiny_prefill_512"), 0)
    dout = I.output_gradient(case, 0)
    check_all(case, dout, run_backward(case, dout))


@pytest.mark.parametrize("branch", [0, 1, 2])
def test_backward_one_branch(branch):
    """Gates one-hot on a branch: each branch's gradient path alone."""
    case = I.generate(I.workload("tiny_prefill_512", seq_len=300), 1)
    case.gates = np.zeros_like(case.gates)
    case.gates[..., branch] = 1.0
    dout = I.output_gradient(case, 1)
    got = run_backward(case, dout)
    check_all(case, dout, got)
    if branch != 0:  # nothing reaches the compressed cache
        assert np.all(got["dkc"] == 0) and np.all(got["dvc"] == 0)


def test_backward_wide_heads_ragged():
    """d_k=192, d_v=128, 16 heads per group, 4 KV heads; 700 positions (ragged against
    every tile: 16-key tiles, 64-key workgroups, 32-position bitmap words, l'=64)."""
    case = I.generate(I.workload("prefill_32k", seq_len=700), 2)
    dout = I.output_gradient(case, 2)
    check_all(case, dout, run_backward(case, dout))


def test_backward_fine_selection_l32():
    case = I.generate(I.workload("prefill_32k", seq_len=400, params={"l_sel": 32, "n_sel": 32}), 3)
    dout = I.output_gradient(case, 3)
    check_all(case, dout, run_backward(case, dout))


def test_backward_shorter_than_one_block():
    """seq_len < l: no compressed block, dk_cmp/dv_cmp absent; the compression
    gradients are exactly zero."""
    case = I.generate(I.workload("tiny_prefill_512", seq_len=20), 4)
    dout = I.output_gradient(case, 4)
    got = run_backward(case, dout)
    check_all(case, dout, got)
    for n in ("dwk", "dpek", "dwv", "dpev"):
        assert np.all(got[n] == 0), n


def test_compress_bwd_repeatable():
    """The compression backward has no atomics: two calls give identical bits."""
    case = I.generate(I.workload("prefill_32k", seq_len=500), 5)
    wl, p = case.wl, case.p
    dims, cfg = U.dims_cfg(case)
    nc = N.compressed_count(wl.seq_len, p.l, p.d)
    rng = np.random.default_rng(5)
    dy = torch.from_numpy(rng.standard_normal((wl.batch, wl.num_kv_heads, nc, wl.d_k), dtype=np.float32)).cuda()
    k = U.dev_bits(case.k)
    outs = []
    for _ in range(2):
        dx = torch.zeros((wl.batch, wl.num_kv_heads, wl.seq_len, wl.d_k), dtype=torch.float32, device="cuda")
        dw = torch.empty((p.l * wl.d_k, wl.d_k), dtype=torch.float32, device="cuda")
        dpe = torch.empty((p.l, wl.d_k), dtype=torch.float32, device="cuda")
        ws = N.new_workspace(N.nsa_compress_bwd_workspace_size(dims, cfg, wl.seq_len, 0))
        N.nsa_compress_bwd(dims, cfg, wl.seq_len, 0, k, U.dev_bits(case.w_k), U.dev_bits(case.pe_k), dy, dx, dw, dpe,
                           ws)
        torch.cuda.synchronize()
        outs.append([t.cpu().numpy() for t in (dx, dw, dpe)])
    for a, b in zip(*outs):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_backward_full_size_samples_and_invariants():
    """prefill_32k at its full size (T=32768), launched as the benchmark launches it.
    dq and dgates of sampled positions against the oracle (one position's terms
    are independent of the others), and sums that hold at any size:
      sum over keys of each branch's dS is 0, so sum_k dk_raw = 0 and sum_i dk_cmp = 0;
      sum over keys of each branch's P is 1, so sum_k dv_raw = sum_t (g_slc + g_win) dout
      and sum_i dv_cmp = sum over positions with a compressed block of g_cmp dout;
      the compression path adds sum_j dPE[j] to the sum of dk over tokens."""
    case = I.generate(I.workload("prefill_32k"), 6)
    wl, p = case.wl, case.p
    T, G = wl.seq_len, wl.num_q_heads // wl.num_kv_heads
    dout = I.output_gradient(case, 6)
    got = run_backward(case, dout)
    rows = [0, 31, 47, 1000, 4095, 17001, T - 1]
    for g in range(wl.num_kv_heads):
        hs = slice(g * G, (g + 1) * G)
        # compared together: at t = 0 every branch has one key, so dq is exactly 0 there
        res = oracle_rows(case, dout, got["sel"], 0, g, rows)
        close(np.stack([got["dq"][0, t, hs] for t in rows]), np.stack([res[t][0] for t in rows]), f"dq g={g}")
        close(np.stack([got["dgates"][0, t, hs] for t in rows]), np.stack([res[t][1] for t in rows]),
              f"dgates g={g}")
    do = _w(dout)[0]                                 # [T, Hq, dv]
    gts = np.asarray(case.gates[0], dtype=np.float64)  # [T, Hq, 3]
    first_cmp = p.l - 1
    for g in range(wl.num_kv_heads):
        hs = slice(g * G, (g + 1) * G)
        sw = ((gts[:, hs, 1:2] + gts[:, hs, 2:3]) * do[:, hs]).sum(axis=(0, 1))
        close(got["dv_raw"][0, g].sum(axis=0, dtype=np.float64), sw, f"sum dv_raw g={g}")
        sc = (gts[first_cmp:, hs, 0:1] * do[first_cmp:, hs]).sum(axis=(0, 1))
        close(got["dvc"][0, g].sum(axis=0, dtype=np.float64), sc, f"sum dv_cmp g={g}")
        for n in ("dk_raw", "dkc"):
            tot = got[n][0, g].astype(np.float64)
            assert np.abs(tot.sum(axis=0)).max() <= 1e-3 * np.abs(tot).sum(axis=0).max(), n
    for x, raw, pe in (("dk", "dk_raw", "dpek"), ("dv", "dv_raw", "dpev")):
        added = (got[x].astype(np.float64) - got[raw]).sum(axis=(0, 1, 2))
        close(added, got[pe].astype(np.float64).sum(axis=0), f"fold vs dPE ({x})")


def test_prefill_bwd_repeatable():
    """Partial sums are combined in a fixed order (no floating-point atomics): two
    backward calls on the same inputs give identical bits."""
    case = I.generate(I.workload("prefill_32k", seq_len=1200), 7)
    dout = I.output_gradient(case, 7)
    a = run_backward(case, dout)
    b = run_backward(case, dout)
    for n in ("dq", "dk", "dv", "dkc", "dvc", "dgates", "dwk", "dpek", "dwv", "dpev"):
        assert np.array_equal(a[n].view(np.uint32), b[n].view(np.uint32)), n


def test_backward_batch_two():
    """Two sequences in one call: every kernel's (sequence, group) indexing."""
    case = I.generate(I.workload("prefill_32k", batch=2, seq_len=333), 8)
    dout = I.output_gradient(case, 8)
    check_all(case, dout, run_backward(case, dout))


@pytest.mark.parametrize("over", [
    dict(num_q_heads=8, num_kv_heads=4, seq_len=260),                                  # G = 2
    dict(seq_len=300, params=dict(l=16, d=8, l_sel=16, n_sel=8, n_local=1)),            # l' = 16
    dict(seq_len=420, params=dict(l_sel=128, n_sel=3, n_local=1)),                     # l' = 128
    dict(seq_len=1),
    dict(seq_len=2),
])
def test_backward_shapes(over):
    """Group sizes that are not a multiple of 4, the smallest and largest selection
    blocks, and sequences of one and two tokens."""
    case = I.generate(I.workload("tiny_prefill_512", **over), 9)
    dout = I.output_gradient(case, 9)
    check_all(case, dout, run_backward(case, dout))


@pytest.mark.parametrize("wl_name,T", [("tiny_prefill_512", 300), ("prefill_32k", 500)])
def test_backward_gate_network(wl_name, T):
    """Gates from the gate network: dq includes the gates' path, and dw_gate,
    db_gate against autograd through the sigmoid layer."""
    case = I.generate(I.workload(wl_name, seq_len=T), 10)
    case.gate_net = True
    dout = I.output_gradient(case, 10)
    got = run_backward(case, dout)
    assert got["dwg"] is not None and got["dbg"] is not None
    check_all(case, dout, got)


@pytest.mark.parametrize("wl_name,T,seed", [("tiny_prefill_512", 512, 11), ("prefill_32k", 700, 12)])
def test_backward_without_saved_lse(wl_name, T, seed):
    """Without the forward's log-sum-exp the query side recomputes each branch's
    softmax in a first pass; same gradients."""
    case = I.generate(I.workload(wl_name, seq_len=T), seed)
    dout = I.output_gradient(case, seed)
    check_all(case, dout, run_backward(case, dout, saved_lse=False))
