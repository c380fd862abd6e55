"""Seeded synthetic inputs for the NSA forward pass (shared by tests, bench and smoke).

This module holds no part of the attention method: it only draws random arrays
with the shapes, scales and planted structure of the workloads, rounds them to
bfloat16 and lays them out in the memory order the C ABI expects.  Both the
CPU oracle and the HIP path receive exactly these arrays.

Workloads follow the NSA parameters of lesson 5.5/02 "Разреженное внимание —
NSA и DSA" (ai.flicky.cc), section "NSA: три ветви" (l=32, d=16, l'=64,
n=16 with the initial and two local blocks, w=512), at the 64k / 128k / 32k
context lengths discussed in its section "Сколько это экономит", and the
needle-in-a-haystack idea of its practice section "«Иголка в стоге сена» на
NumPy" (a block of keys pointing along the query direction).

Draw order for every workload (one ``numpy.random.default_rng(seed)`` stream):
  1. per-sequence lengths (ragged workloads only)
  2. q, k, v                    ~ scale * N(0, 1)
  3. gate pre-activations z     ~ N(0, 1); gate values = sigmoid(z)
  4. W_k, PE_k, W_v, PE_v       W ~ N(0, 1/(l*D)), PE ~ N(0, 0.02^2)
  5. needle block positions     uniform without replacement over non-forced blocks
  6. needle noise               keys of needle tokens = scale*(sqrt(dk)*u + 0.1*eps)
  7. gate-network weights       W_gate ~ N(0, 1/dk)/scale (unit-variance pre-activations),
                                b_gate ~ N(0, 0.5^2); used only by cases with gate_net set
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass, field
from typing import Optional

import numpy as np


@dataclass(frozen=True)
class NSAParams:
    l: int            # compression block length
    d: int            # compression stride
    l_sel: int        # selection block length (l')
    n_sel: int        # selected blocks per (query, KV group), forced ones included
    n_local: int      # trailing (local) blocks always selected
    force_initial: int  # 1: block 0 always selected
    w: int            # sliding-window length


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str                 # "prefill" or "decode"
    batch: int
    num_q_heads: int
    num_kv_heads: int
    d_k: int
    d_v: int
    seq_len: int              # prefill length N, or decode context length L (max for ragged)
    params: NSAParams
    needles: int              # planted needle blocks per (sequence, KV head)
    scale: float = 1.0        # multiplier on q, k, v
    ragged_min: Optional[int] = None   # ragged decode: lengths ~ U{ragged_min .. seq_len}
    description: str = ""

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


_STD = NSAParams(l=32, d=16, l_sel=64, n_sel=16, n_local=2, force_initial=1, w=512)

WORKLOADS = {
    "tiny_prefill_512": Workload(
        "tiny_prefill_512", "prefill", 1, 4, 1, 64, 64, 512,
        NSAParams(l=32, d=16, l_sel=64, n_sel=4, n_local=1, force_initial=1, w=64),
        needles=3, description="tiny prefill, N=512, 4 q heads / 1 KV head, d=64"),
    "decode_64k_b8": Workload(
        "decode_64k_b8", "decode", 8, 64, 4, 192, 128, 65536, _STD, needles=8,
        description="decode step, batch 8, 64k context, 64q/4kv heads, dk=192, dv=128"),
    "prefill_32k": Workload(
        "prefill_32k", "prefill", 1, 64, 4, 192, 128, 32768, _STD, needles=8, scale=0.5,
        description="causal prefill, N=32768, 64q/4kv heads, dk=192, dv=128"),
    "decode_128k_b4": Workload(
        "decode_128k_b4", "decode", 4, 64, 4, 192, 128, 131072, _STD, needles=16,
        description="decode step, batch 4, 128k context"),
    "decode_ragged_16": Workload(
        "decode_ragged_16", "decode", 16, 64, 4, 192, 128, 65536,
        NSAParams(l=32, d=16, l_sel=32, n_sel=32, n_local=2, force_initial=1, w=512),
        needles=8, ragged_min=4096,
        description="ragged decode, 16 sequences of 4096..65536 tokens, l'=32, n=32"),
}


# --------------------------------------------------------------------------- bf16

def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round-to-nearest-even); return uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _round(x):
    return bf16_bits(x)


# --------------------------------------------------------------------------- cases

@dataclass
class Case:
    """One seeded instance.  bf16 tensors are held as uint16 bit patterns.

    Prefill layouts: q [B,T,Hq,dk], k [B,Hkv,T,dk], v [B,Hkv,T,dv], gates [B,T,Hq,3].
    Decode layouts:  q [B,Hq,dk], gates [B,Hq,3]; k/v caches are packed row arrays
    [sum_b Hkv*cap_b, D] where sequence b, head g, token x lives at row
    Hkv*cu_seqlens[b] + g*cap_b + x and cap_b = cu_seqlens[b+1]-cu_seqlens[b].
    """
    wl: Workload
    seed: int
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    gates: np.ndarray
    w_k: np.ndarray
    pe_k: np.ndarray
    w_v: np.ndarray
    pe_v: np.ndarray
    seq_lens: Optional[np.ndarray] = None     # decode: int32 [B], includes the current token
    cu_seqlens: Optional[np.ndarray] = None   # decode: int64 [B+1] token-capacity offsets
    needle_blocks: list = field(default_factory=list)  # per (b, g): list of l'-block ids
    w_gate: Optional[np.ndarray] = None       # gate network weights [Hq, 3, dk] (bf16 bits)
    b_gate: Optional[np.ndarray] = None       # gate network bias [Hq, 3] (float32)
    gate_net: bool = False                    # True: the gates come from the gate network
    fp32: Optional[dict] = None               # unrounded float32 copies (small workloads only)

    @property
    def p(self) -> NSAParams:
        return self.wl.params

    def f32(self, name: str) -> np.ndarray:
        return bits_to_f32(getattr(self, name))

    # decode cache helpers (row offsets only; no arithmetic of the method)
    def kv_rows(self, b: int, g: int):
        H = self.wl.num_kv_heads
        cu = self.cu_seqlens
        cap = int(cu[b + 1] - cu[b])
        start = H * int(cu[b]) + g * cap
        return start, int(self.seq_lens[b])


def _needle_direction(qg: np.ndarray) -> np.ndarray:
    """Unit vector along the mean of the given query vectors (rows)."""
    m = qg.reshape(-1, qg.shape[-1]).astype(np.float64).mean(axis=0)
    return m / np.linalg.norm(m)


def _non_forced_blocks(L: int, p: NSAParams) -> np.ndarray:
    J = (L - 1) // p.l_sel
    forced = set(range(J - p.n_local + 1, J + 1))
    if p.force_initial:
        forced.add(0)
    return np.array([j for j in range(J + 1) if j not in forced], dtype=np.int64)


def generate(wl: Workload, seed: int, keep_fp32: bool = False) -> Case:
    """Draw one seeded case of workload ``wl`` (see the module docstring for the order)."""
    rng = np.random.default_rng(seed)
    p = wl.params
    B, Hq, H, dk, dv = wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.d_k, wl.d_v
    G = Hq // H
    s = np.float32(wl.scale)

    # 1. lengths
    if wl.kind == "decode":
        if wl.ragged_min is not None:
            lens = rng.integers(wl.ragged_min, wl.seq_len + 1, size=B).astype(np.int64)
        else:
            lens = np.full(B, wl.seq_len, dtype=np.int64)
    else:
        lens = np.full(B, wl.seq_len, dtype=np.int64)

    # 2. q, k, v
    def normal(shape):
        return rng.standard_normal(size=shape, dtype=np.float32)

    if wl.kind == "prefill":
        T = wl.seq_len
        q = normal((B, T, Hq, dk)) * s
        k = normal((B, H, T, dk)) * s
        v = normal((B, H, T, dv)) * s
    else:
        total = int(lens.sum())
        q = normal((B, Hq, dk)) * s
        k = normal((H * total, dk)) * s
        v = normal((H * total, dv)) * s

    # 3. gates
    z = rng.standard_normal(size=(q.shape[:-1] + (3,))).astype(np.float64)
    gates = (1.0 / (1.0 + np.exp(-z))).astype(np.float32)

    # 4. compression weights and intra-block position embeddings
    w_k = rng.standard_normal(size=(p.l * dk, dk), dtype=np.float32) / np.float32(np.sqrt(p.l * dk))
    pe_k = rng.standard_normal(size=(p.l, dk), dtype=np.float32) * np.float32(0.02)
    w_v = rng.standard_normal(size=(p.l * dv, dv), dtype=np.float32) / np.float32(np.sqrt(p.l * dv))
    pe_v = rng.standard_normal(size=(p.l, dv), dtype=np.float32) * np.float32(0.02)

    # 5./6. needles
    cu = np.zeros(B + 1, dtype=np.int64)
    cu[1:] = np.cumsum(lens)
    needle_blocks = []
    for b in range(B):
        L = int(lens[b])
        cand = _non_forced_blocks(L, p)
        for g in range(H):
            cnt = min(wl.needles, len(cand))
            picks = np.sort(rng.choice(cand, size=cnt, replace=False)) if cnt else np.zeros(0, np.int64)
            needle_blocks.append(picks)
    noises = []
    for b in range(B):
        L = int(lens[b])
        for g in range(H):
            picks = needle_blocks[b * H + g]
            rows = []
            for j in picks:
                lo, hi = int(j) * p.l_sel, min((int(j) + 1) * p.l_sel, L)
                rows.append(np.arange(lo, hi))
            rows = np.concatenate(rows) if rows else np.zeros(0, np.int64)
            eps = rng.standard_normal(size=(rows.size, dk), dtype=np.float32)
            noises.append((rows, eps))
    for b in range(B):
        for g in range(H):
            rows, eps = noises[b * H + g]
            if rows.size == 0:
                continue
            if wl.kind == "prefill":
                u = _needle_direction(q[b, :, g * G:(g + 1) * G, :])
                k[b, g, rows, :] = s * (np.float32(np.sqrt(dk)) * u.astype(np.float32) + np.float32(0.1) * eps)
            else:
                u = _needle_direction(q[b, g * G:(g + 1) * G, :])
                start = H * int(cu[b]) + g * int(lens[b])
                k[start + rows, :] = s * (np.float32(np.sqrt(dk)) * u.astype(np.float32) + np.float32(0.1) * eps)

    fp32 = None
    if keep_fp32:
        fp32 = dict(q=q.copy(), k=k.copy(), v=v.copy(), w_k=w_k.copy(), pe_k=pe_k.copy(),
                    w_v=w_v.copy(), pe_v=pe_v.copy())
    # 7. gate-network weights (drawn last, so every earlier value is unchanged):
    #    w_gate [Hq, 3, dk] ~ N(0, 1/dk) / scale, b_gate [Hq, 3] ~ N(0, 0.5^2)
    w_gate = rng.standard_normal(size=(Hq, 3, dk), dtype=np.float32) / np.float32(np.sqrt(dk) * s)
    b_gate = (rng.standard_normal(size=(Hq, 3), dtype=np.float32) * np.float32(0.5))

    case = Case(wl=wl, seed=seed, q=_round(q), k=_round(k), v=_round(v), gates=gates,
                w_k=_round(w_k), pe_k=_round(pe_k), w_v=_round(w_v), pe_v=_round(pe_v),
                needle_blocks=needle_blocks, fp32=fp32, w_gate=_round(w_gate), b_gate=b_gate)
    if wl.kind == "decode":
        case.seq_lens = lens.astype(np.int32)
        case.cu_seqlens = cu
    return case


def output_gradient(case: Case, seed: int) -> np.ndarray:
    """Seeded gradient of a prefill case's output for the backward pass: bf16 bits
    [B, T, Hq, d_v] of standard normal values, drawn from its own stream
    default_rng([seed, 1]) so that the forward inputs do not change."""
    wl = case.wl
    rng = np.random.default_rng([seed, 1])
    g = rng.standard_normal(size=(wl.batch, wl.seq_len, wl.num_q_heads, wl.d_v), dtype=np.float32)
    return bf16_bits(g)


def workload(name: str, **overrides) -> Workload:
    wl = WORKLOADS[name]
    if "params" in overrides and isinstance(overrides["params"], dict):
        overrides["params"] = dataclasses.replace(wl.params, **overrides["params"])
    return wl.with_(**overrides) if overrides else wl



# --------------------------------------------------------------------------- DSA decode workloads
#
# DeepSeek Sparse Attention as described in lesson 5.5/02 (section "DSA:
# молниеносный индексатор"): an FP8 lightning indexer with a few small heads,
# 2048 selected tokens per query, MLA in MQA mode over one 576-number latent per
# token (512 of them the values).  Draw order (one default_rng(seed) stream):
#   1. lengths (ragged workloads only)
#   2. q [B, H, 576], latent c [B, cap, 576]      ~ N(0, 1), rounded to bf16
#   3. q_idx [B, HI, DI], k_idx [B, cap, DI]      ~ N(0, 1), rounded to FP8 E4M3
#   4. w_idx [B, HI]                              ~ N(0, 1/HI)
#   5. needles: positions uniform without replacement over [0, L_b); their
#      indexer keys point along sum_j max(w_j, 0) q_idx_j (length 2 sqrt(DI)) and
#      their latents along the mean query (length sqrt(576)), plus 0.1 noise


@dataclass(frozen=True)
class DsaWorkload:
    name: str
    batch: int
    num_heads: int
    d_qk: int
    d_v: int
    idx_heads: int
    idx_dim: int
    top_k: int
    seq_len: int              # cache length per sequence (the largest length)
    needles: int
    ragged_min: Optional[int] = None
    kind: str = "dsa_decode"
    description: str = ""

    def with_(self, **kw) -> "DsaWorkload":
        return dataclasses.replace(self, **kw)


DSA_WORKLOADS = {
    "dsa_decode_64k_b8": DsaWorkload(
        "dsa_decode_64k_b8", 8, 128, 576, 512, 16, 128, 2048, 65536, 32,
        description="DSA decode step, batch 8, 64k context, 128 heads over a 576-number latent, "
                    "16 x 128 FP8 indexer heads, top-2048"),
}


def fp8_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to FP8 E4M3 (OCP, round to nearest even); uint8 bit patterns."""
    import torch
    t = torch.from_numpy(np.clip(np.ascontiguousarray(x, dtype=np.float32), -448.0, 448.0))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


@dataclass
class DsaCase:
    wl: DsaWorkload
    seed: int
    q: np.ndarray           # bf16 bits [B, H, d_qk]
    c: np.ndarray           # bf16 bits [B, cap, d_qk]
    q_idx: np.ndarray       # FP8 bits [B, HI, DI]
    k_idx: np.ndarray       # FP8 bits [B, cap, DI]
    w_idx: np.ndarray       # float32 [B, HI]
    seq_lens: np.ndarray    # int32 [B]
    needle_pos: list = field(default_factory=list)


def generate_dsa(wl: DsaWorkload, seed: int) -> DsaCase:
    rng = np.random.default_rng(seed)
    B, H, D, HI, DI, cap = wl.batch, wl.num_heads, wl.d_qk, wl.idx_heads, wl.idx_dim, wl.seq_len
    if wl.ragged_min is not None:
        lens = rng.integers(wl.ragged_min, cap + 1, size=B).astype(np.int64)
    else:
        lens = np.full(B, cap, dtype=np.int64)
    q = rng.standard_normal(size=(B, H, D), dtype=np.float32)
    c = rng.standard_normal(size=(B, cap, D), dtype=np.float32)
    q_idx = rng.standard_normal(size=(B, HI, DI), dtype=np.float32)
    k_idx = rng.standard_normal(size=(B, cap, DI), dtype=np.float32)
    w_idx = (rng.standard_normal(size=(B, HI), dtype=np.float32) / np.float32(np.sqrt(HI)))
    needle_pos = []
    for b in range(B):
        L = int(lens[b])
        cnt = min(wl.needles, L)
        pos = np.sort(rng.choice(L, size=cnt, replace=False)) if cnt else np.zeros(0, np.int64)
        needle_pos.append(pos)
        if cnt == 0:
            continue
        ui = (np.maximum(w_idx[b], 0.0)[:, None] * q_idx[b]).sum(axis=0)
        ui = ui / max(np.linalg.norm(ui), 1e-6)
        uq = q[b].mean(axis=0)
        uq = uq / np.linalg.norm(uq)
        k_idx[b, pos] = (2.0 * np.sqrt(DI) * ui)[None, :] + 0.1 * rng.standard_normal((cnt, DI), dtype=np.float32)
        c[b, pos] = (np.sqrt(D) * uq)[None, :] + 0.1 * rng.standard_normal((cnt, D), dtype=np.float32)
    return DsaCase(wl=wl, seed=seed, q=_round(q), c=_round(c), q_idx=fp8_bits(q_idx), k_idx=fp8_bits(k_idx),
                   w_idx=w_idx, seq_lens=lens.astype(np.int32), needle_pos=needle_pos)


def dsa_workload(name: str, **overrides) -> DsaWorkload:
    wl = DSA_WORKLOADS[name]
    return wl.with_(**overrides) if overrides else wl
