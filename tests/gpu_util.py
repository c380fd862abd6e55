"""Helpers for the GPU parity tests: upload seeded cases, call the C ABI, compare.

Tolerances (bf16 in, fp32 accumulate): outputs max-abs <= 2e-2 and mean-abs
<= 2e-3 against the float64 oracle; selected block sets identical except where
the oracle's gap between the last routed pick and the next candidate is below
1e-3 relative, in which case the GPU's set must still be a valid top-n within
that gap and its output must match the oracle re-run on the GPU's set.
"""
from __future__ import annotations

import numpy as np
import torch

import long_context_sparse_nsa_amd as N
from oracle import nsa_oracle as O

MAX_ABS = 2e-2
MEAN_ABS = 2e-3
TIE_REL = 1e-3


def dev_bits(a: np.ndarray) -> torch.Tensor:
    """uint16 bf16 bit patterns -> torch.bfloat16 tensor on the GPU."""
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def host_bits(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def bits_to_f64(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def dims_cfg(case):
    wl, p = case.wl, case.p
    dims = N.make_dims(wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.d_k, wl.d_v)
    cfg = N.make_config(p.l, p.d, p.l_sel, p.n_sel, p.n_local, p.force_initial, p.w)
    return dims, cfg


def cmp_offsets(case) -> np.ndarray:
    """Row offsets of a packed compressed cache sized to each sequence's capacity."""
    p = case.p
    caps = np.diff(case.cu_seqlens)
    ncap = np.array([N.compressed_count(int(c), p.l, p.d) for c in caps], dtype=np.int64)
    out = np.zeros(len(caps) + 1, dtype=np.int64)
    out[1:] = np.cumsum(ncap)
    return out


def oracle_cmp_cache(case, groups=None):
    """Oracle compressed cache of every (b, g), packed like cmp_offsets; bf16 bits."""
    wl = case.wl
    H = wl.num_kv_heads
    cuc = cmp_offsets(case)
    kc = np.zeros((int(H * cuc[-1]), wl.d_k), dtype=np.uint16)
    vc = np.zeros((int(H * cuc[-1]), wl.d_v), dtype=np.uint16)
    for b in range(wl.batch):
        ccap = int(cuc[b + 1] - cuc[b])
        for g in range(H):
            _, _, Kc, Vc = O.compress_group(case, b, g)
            r0 = H * int(cuc[b]) + g * ccap
            kc[r0:r0 + Kc.shape[0]] = f64_to_bits(Kc)
            vc[r0:r0 + Vc.shape[0]] = f64_to_bits(Vc)
    return kc, vc, cuc


def f64_to_bits(x: np.ndarray) -> np.ndarray:
    """Exact bf16 values (float64) -> bit patterns."""
    return (np.asarray(x, dtype=np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def run_decode(case, kc_bits=None, vc_bits=None, gates=None, ws=None, max_len=None):
    """Decode step on the GPU.  Without kc/vc the GPU compresses the cache first.
    max_len (default: the largest capacity) also sets the launch plan."""
    wl = case.wl
    dims, cfg = dims_cfg(case)
    cuc = cmp_offsets(case)
    q = dev_bits(case.q)
    k = dev_bits(case.k)
    v = dev_bits(case.v)
    seq = torch.from_numpy(case.seq_lens).cuda()
    cu = torch.from_numpy(case.cu_seqlens).cuda()
    cu_c = torch.from_numpy(cuc).cuda()
    cap_max = int(np.diff(case.cu_seqlens).max())
    max_len = cap_max if max_len is None else int(max_len)
    if kc_bits is None:
        rows = int(wl.num_kv_heads * cuc[-1])
        kc = torch.zeros((max(rows, 1), wl.d_k), dtype=torch.bfloat16, device="cuda")
        vc = torch.zeros((max(rows, 1), wl.d_v), dtype=torch.bfloat16, device="cuda")
        N.nsa_compress_kv(dims, cfg, k, v, cu, seq, cap_max, dev_bits(case.w_k), dev_bits(case.pe_k),
                          dev_bits(case.w_v), dev_bits(case.pe_v), kc, vc, cu_c)
    else:
        if kc_bits.shape[0] == 0:  # no complete block yet: the cache is never read, but must not be NULL
            kc_bits = np.zeros((1, wl.d_k), np.uint16)
            vc_bits = np.zeros((1, wl.d_v), np.uint16)
        kc, vc = dev_bits(kc_bits), dev_bits(vc_bits)
    g, wg, bgt = gate_args(case, gates)
    out = torch.empty((wl.batch, wl.num_q_heads, wl.d_v), dtype=torch.bfloat16, device="cuda")
    sel = torch.full((wl.batch, wl.num_kv_heads, cfg.n_sel), -7, dtype=torch.int32, device="cuda")
    if ws is None:
        ws = N.new_workspace(N.nsa_decode_workspace_size(dims, cfg, max_len))
    N.nsa_decode_fwd(dims, cfg, q, k, v, kc, vc, seq, cu, cu_c, max_len, g, out, sel, ws, w_gate=wg, b_gate=bgt)
    torch.cuda.synchronize()
    return bits_to_f64(host_bits(out)), sel.cpu().numpy(), (kc, vc)


def gate_args(case, gates=None):
    """(gates, w_gate, b_gate) device arguments: the gate network's weights when the
    case sets gate_net, else the gate values."""
    if getattr(case, "gate_net", False):
        bgt = torch.from_numpy(np.ascontiguousarray(case.b_gate, dtype=np.float32)).cuda() \
            if case.b_gate is not None else None
        return None, dev_bits(case.w_gate), bgt
    g = torch.from_numpy(np.ascontiguousarray(case.gates if gates is None else gates, dtype=np.float32)).cuda()
    return g, None, None


def run_prefill(case, gates=None, kc_bits=None, vc_bits=None, with_lse=False):
    wl = case.wl
    dims, cfg = dims_cfg(case)
    T = wl.seq_len
    g, wg, bgt = gate_args(case, gates)
    out = torch.empty((wl.batch, T, wl.num_q_heads, wl.d_v), dtype=torch.bfloat16, device="cuda")
    sel = torch.full((wl.batch, T, wl.num_kv_heads, cfg.n_sel), -7, dtype=torch.int32, device="cuda")
    lse = (torch.full((wl.batch, T, wl.num_q_heads, 3), float("nan"), dtype=torch.float32, device="cuda")
           if with_lse else None)
    compress = kc_bits is None
    ws = N.new_workspace(N.nsa_prefill_workspace_size(dims, cfg, T, compress))
    kc = None if compress else dev_bits(kc_bits)
    vc = None if compress else dev_bits(vc_bits)
    N.nsa_prefill_fwd(dims, cfg, T, dev_bits(case.q), dev_bits(case.k), dev_bits(case.v), kc, vc,
                      dev_bits(case.w_k), dev_bits(case.pe_k), dev_bits(case.w_v), dev_bits(case.pe_v),
                      g, out, sel, ws, w_gate=wg, b_gate=bgt, lse_out=lse)
    torch.cuda.synchronize()
    if with_lse:
        return bits_to_f64(host_bits(out)), sel.cpu().numpy(), lse.cpu().numpy()
    return bits_to_f64(host_bits(out)), sel.cpu().numpy()


# ------------------------------------------------------------------ comparison

def tie_gap(res: O.QueryResult, t: int, p) -> float:
    """Relative gap between the last routed pick and the first unpicked candidate."""
    J = t // p.l_sel
    if J + 1 <= p.n_sel:
        return np.inf
    F = set(O.forced_blocks(J, p.n_local, p.force_initial))
    rest = sorted((j for j in range(J + 1) if j not in F), key=lambda j: (-res.scores[j], j))
    nr = p.n_sel - len(F)
    if nr <= 0 or nr >= len(rest):
        return np.inf
    a, b = res.scores[rest[nr - 1]], res.scores[rest[nr]]
    return (a - b) / a if a > 0 else 0.0


def check_selection(res: O.QueryResult, gpu_idx, t: int, p, rerun):
    """Compare one (query, group) selection.  Returns the oracle result to compare outputs with."""
    got = [int(j) for j in gpu_idx if j >= 0]
    assert all(j == -1 for j in gpu_idx[len(got):]), f"padding broken: {gpu_idx}"
    if got == res.idx:
        return res
    gap = tie_gap(res, t, p)
    assert gap < TIE_REL, f"t={t}: GPU picked {got}, oracle {res.idx} (gap {gap:.3g})"
    J = t // p.l_sel
    F = set(O.forced_blocks(J, p.n_local, p.force_initial))
    assert F <= set(got) and len(got) == len(res.idx) and got == sorted(got) and max(got) <= J
    thr = min(res.scores[j] for j in res.idx if j not in F)
    for j in set(got) - F:
        assert res.scores[j] >= thr * (1 - 2 * TIE_REL), f"t={t}: GPU routed block {j} is not near the top"
    return rerun(got)


def assert_close(got: np.ndarray, want: np.ndarray, what: str):
    err = np.abs(got - want)
    assert err.max() <= MAX_ABS, f"{what}: max-abs {err.max():.4g} > {MAX_ABS}"
    assert err.mean() <= MEAN_ABS, f"{what}: mean-abs {err.mean():.4g} > {MEAN_ABS}"
    return float(err.max()), float(err.mean())
