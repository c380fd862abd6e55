"""Plain float64 CPU oracle of the Native Sparse Attention (NSA) forward pass.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the CPU
baseline leg of the benchmark may import this module; the library never does.
It shares no code with the HIP path.

Sources (page title, then section / equation / table):
  [LES]  Lesson "Native Sparse Attention (DeepSeek NSA)", AI Engineering from
         Scratch, phase 10 · 17 (Hindi): sections "Concept — three parallel
         branches", "Compute budget", "Build it" (steps 1-6), "Key terms".
  [FLI]  Lesson 5.5/02 "Разреженное внимание — NSA и DSA" (ai.flicky.cc):
         section "NSA: три ветви" (output equation and the three branch
         paragraphs), "Сколько это экономит" (read-count table), practice
         "Задание в браузере" (window / top-k / masked-attention spec).

What is computed for one query position t and one KV group g (G query heads):

  compression   kc_i = flatten(K[i*d : i*d+l] + PE_k) . W_k, same for values;
                rounded to bfloat16 because the compressed cache is bf16.
                [FLI "NSA: три ветви", compressed-branch paragraph: blocks of
                l=32 tokens, stride d=16, a learned MLP folds each block into one
                key and one value.]  The MLP is read as one bias-free linear layer
                on the flattened block plus a learned intra-block position
                embedding.
  visibility    compressed block i is visible to t iff its last token i*d+l-1 <= t.
  cmp branch    softmax(s * q.kc) over visible blocks, times vc; zero if none.
  scores        per head the branch probabilities are folded onto selection
                blocks of l' tokens with weight |block_i ∩ sel_j| / l, then summed
                over the heads of the group [FLI selection paragraph: the weights
                are re-counted onto larger l'=64 blocks; all heads of a GQA group
                pick the same blocks].
  top-n         the initial block and the n_local trailing blocks are always
                taken and count toward n; the rest are the highest group scores,
                ties to the lower block index; if at most n blocks exist, all are
                taken [FLI selection paragraph; practice spec: "if fewer than k
                keys, take all", never the future].
  slc branch    softmax attention over the tokens of the selected blocks, x <= t.
  win branch    softmax attention over tokens x with x <= t and t - x < w
                [FLI practice spec of sliding_window_mask].
  combine       out = g_cmp*o_cmp + g_slc*o_slc + g_win*o_win with the gate values
                as given (they need not sum to one) [FLI output equation; LES
                "Concept"], or computed from each head's query by the gate
                network: sigmoid of one linear layer [LES "Build it" step 5].
  attention     scale 1/sqrt(d_k), forbidden pairs excluded, row-max-subtracted
                softmax [FLI practice spec of sparse_attention].
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np


# --------------------------------------------------------------------------- helpers

def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 value (ties to even), returned as float64.

    The compressed key/value cache is stored in bfloat16, so the oracle's
    compressed keys/values take the same rounding step once.  Splits x into
    mantissa and exponent, rounds the mantissa to 8 significant bits (bf16 has
    8 including the implicit one) half-to-even, and scales back; every step is
    exact in float64.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.empty_like(x)
    flat = x.reshape(-1)
    res = out.reshape(-1)
    m, e = np.frexp(flat)                   # flat = m * 2**e, 0.5 <= |m| < 1
    scaled = np.ldexp(m, 8)                 # 8 significant bits before the point
    r = np.round(scaled)                    # numpy rounds half to even
    res[:] = np.ldexp(r, e - 8)
    res[flat == 0] = 0.0
    return out


def n_compressed(L: int, l: int, d: int) -> int:
    """Number of complete compression blocks among the first L tokens."""
    return (L - l) // d + 1 if L >= l else 0


# --------------------------------------------------------------------------- a1 compression

def compress(Kseq: np.ndarray, W: np.ndarray, PE: np.ndarray, l: int, d: int,
             round_bf16: bool = True) -> np.ndarray:
    """Compressed keys (or values) of one sequence and head.

    Kseq [L, D], W [l*D, D], PE [l, D].  Block i covers tokens [i*d, i*d+l);
    its summary is (K[block] + PE) flattened token-major, times W.
    [FLI "NSA: три ветви", compressed branch; LES "Build it" step 1.]
    """
    L, D = Kseq.shape
    nc = n_compressed(L, l, d)
    if nc == 0:
        return np.zeros((0, W.shape[1]), dtype=np.float64)
    K64 = np.asarray(Kseq, dtype=np.float64)
    X = np.stack([(K64[i * d:i * d + l] + PE).reshape(-1) for i in range(nc)])
    out = X @ np.asarray(W, dtype=np.float64)
    return round_to_bf16(out) if round_bf16 else out


# --------------------------------------------------------------------------- attention primitive

def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float):
    """Softmax attention of query rows q [H, dk] over keys K [n, dk], values V [n, dv].

    Returns (out [H, dv], probs [H, n]); with n == 0 the output is zero.
    [FLI practice, sparse_attention: scale 1/sqrt(d), row-max-subtracted softmax.]
    """
    q = np.atleast_2d(np.asarray(q, dtype=np.float64))
    H = q.shape[0]
    if K.shape[0] == 0:
        return np.zeros((H, V.shape[1])), np.zeros((H, 0))
    z = scale * (q @ np.asarray(K, dtype=np.float64).T)
    z = z - z.max(axis=1, keepdims=True)
    e = np.exp(z)
    p = e / e.sum(axis=1, keepdims=True)
    return p @ np.asarray(V, dtype=np.float64), p


def log_sum_exp(q: np.ndarray, K: np.ndarray, scale: float) -> np.ndarray:
    """Natural log of sum_k exp(scale * q . k) for each query row q [H, dk] over
    keys K [n, dk] -- the normaliser of the softmax in `attend`; -inf when n == 0."""
    q = np.atleast_2d(np.asarray(q, dtype=np.float64))
    if K.shape[0] == 0:
        return np.full(q.shape[0], -np.inf)
    z = scale * (q @ np.asarray(K, dtype=np.float64).T)
    m = z.max(axis=1)
    return m + np.log(np.exp(z - m[:, None]).sum(axis=1))


# --------------------------------------------------------------------------- a2 fold + top-n

def fold_weights(n_keys: int, l: int, d: int, l_sel: int, n_blocks: int) -> np.ndarray:
    """omega[i, j] = |[i*d, i*d+l) ∩ [j*l', (j+1)*l')| / l  (token-overlap share).

    Re-counts compressed-block weights onto selection blocks of l' tokens
    [FLI "NSA: три ветви", selection paragraph].
    """
    om = np.zeros((n_keys, n_blocks))
    for i in range(n_keys):
        a0, a1 = i * d, i * d + l
        for j in range(a0 // l_sel, min(n_blocks, (a1 - 1) // l_sel + 1)):
            b0, b1 = j * l_sel, (j + 1) * l_sel
            ov = min(a1, b1) - max(a0, b0)
            if ov > 0:
                om[i, j] = ov / l
    return om


def forced_blocks(J: int, n_local: int, force_initial: int) -> list:
    """Blocks always selected at a query whose own block is J: block 0 and J, J-1, ..."""
    f = set()
    if force_initial:
        f.add(0)
    for r in range(n_local):
        if J - r >= 0:
            f.add(J - r)
    return sorted(f)


def select_blocks(S: np.ndarray, J: int, n: int, n_local: int, force_initial: int) -> list:
    """Top-n selection over candidate blocks 0..J with group scores S[0..J].

    Forced blocks count toward n; remaining slots go to the highest scores,
    equal scores to the lower index; if J+1 <= n every candidate is taken.
    Returned ascending.
    """
    if J + 1 <= n:
        return list(range(J + 1))
    F = forced_blocks(J, n_local, force_initial)
    rest = [j for j in range(J + 1) if j not in F]
    rest.sort(key=lambda j: (-S[j], j))
    return sorted(F + rest[:n - len(F)])


# --------------------------------------------------------------------------- gate network

def gate_network(qg: np.ndarray, Wg: np.ndarray, bg: Optional[np.ndarray]) -> np.ndarray:
    """Branch gates of G query heads from their query vectors.

    qg [G, dk]; Wg [G, 3, dk] (head h's three weight rows, in the order cmp,
    slc, win); bg [G, 3] or None.  gate[h, c] = sigmoid(Wg[h, c] . qg[h] + bg[h, c]).
    [LES "Build it" step 5: a small MLP on the query yields the three gate
    weights; FLI "NSA: три ветви": gates in [0, 1] from a small network with a
    sigmoid.]  The small network is read as one linear layer with a bias.
    """
    q = np.asarray(qg, dtype=np.float64)
    W = np.asarray(Wg, dtype=np.float64)
    z = np.einsum("hck,hk->hc", W, q)
    if bg is not None:
        z = z + np.asarray(bg, dtype=np.float64)
    return 1.0 / (1.0 + np.exp(-z))


# --------------------------------------------------------------------------- one query

@dataclass
class QueryResult:
    out: np.ndarray          # [G, dv]
    o_cmp: np.ndarray
    o_slc: np.ndarray
    o_win: np.ndarray
    idx: list                # selected blocks, ascending
    scores: np.ndarray       # group scores S[0..J]
    lse: np.ndarray = None   # [G, 3] each branch's log-sum-exp (cmp, slc, win), natural log


def nsa_query(qg: np.ndarray, K: np.ndarray, V: np.ndarray, Kc: np.ndarray, Vc: np.ndarray,
              t: int, gates: np.ndarray, l: int, d: int, l_sel: int, n: int, n_local: int,
              force_initial: int, w: int, scale: Optional[float] = None,
              override_idx: Optional[Sequence[int]] = None) -> QueryResult:
    """NSA output of the G query heads qg [G, dk] of one KV group at position t.

    K [>=t+1, dk], V: the group's raw cache; Kc/Vc: its compressed cache (at least
    the blocks visible at t).  gates [G, 3] = (g_cmp, g_slc, g_win).
    ``override_idx`` recomputes the selected branch and output for a given block set.
    """
    qg = np.asarray(qg, dtype=np.float64)
    dk = qg.shape[1]
    s = 1.0 / np.sqrt(dk) if scale is None else scale
    # compressed branch over visible blocks
    nvis = n_compressed(t + 1, l, d)
    o_cmp, p = attend(qg, Kc[:nvis], Vc[:nvis], s)
    # group scores on selection blocks
    J = t // l_sel
    S = (p @ fold_weights(nvis, l, d, l_sel, J + 1)).sum(axis=0) if nvis else np.zeros(J + 1)
    idx = list(override_idx) if override_idx is not None else select_blocks(S, J, n, n_local, force_initial)
    # selected branch
    toks = np.concatenate([np.arange(j * l_sel, min((j + 1) * l_sel, t + 1)) for j in idx])
    o_slc, _ = attend(qg, K[toks], V[toks], s)
    # sliding window
    wt = np.arange(max(0, t - w + 1), t + 1)
    o_win, _ = attend(qg, K[wt], V[wt], s)
    g = np.asarray(gates, dtype=np.float64)
    out = g[:, 0:1] * o_cmp + g[:, 1:2] * o_slc + g[:, 2:3] * o_win
    lse = np.stack([log_sum_exp(qg, Kc[:nvis], s), log_sum_exp(qg, K[toks], s), log_sum_exp(qg, K[wt], s)], axis=1)
    return QueryResult(out, o_cmp, o_slc, o_win, idx, S, lse)


# --------------------------------------------------------------------------- batch drivers

def _widen(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float64 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def _group_gates(case, qg, g: int, G: int, given):
    """The gates of one position's group heads: computed by the gate network when
    the case says so (case.gate_net), else the given values."""
    if getattr(case, "gate_net", False):
        Wg = _widen(case.w_gate[g * G:(g + 1) * G])
        bg = None if case.b_gate is None else np.asarray(case.b_gate[g * G:(g + 1) * G], dtype=np.float64)
        return gate_network(qg, Wg, bg)
    return np.asarray(given, dtype=np.float64)


def compress_group(case, b: int, g: int, upto: Optional[int] = None):
    """Oracle compressed cache (bf16-rounded, float64) of sequence b, KV head g."""
    p = case.wl.params
    if case.wl.kind == "prefill":
        K = _widen(case.k[b, g])
        V = _widen(case.v[b, g])
    else:
        start, L = case.kv_rows(b, g)
        K = _widen(case.k[start:start + L])
        V = _widen(case.v[start:start + L])
    if upto is not None:
        K, V = K[:upto], V[:upto]
    Kc = compress(K, _widen(case.w_k), _widen(case.pe_k), p.l, p.d)
    Vc = compress(V, _widen(case.w_v), _widen(case.pe_v), p.l, p.d)
    return K, V, Kc, Vc


def decode_group(case, b: int, g: int, Kc=None, Vc=None, override_idx=None) -> QueryResult:
    """Decode step of sequence b, KV group g: the query sits at t = seq_len - 1.

    Kc/Vc default to the oracle's own compression of the group's cache.
    """
    p = case.wl.params
    G = case.wl.num_q_heads // case.wl.num_kv_heads
    K, V, Kc_o, Vc_o = compress_group(case, b, g)
    if Kc is None:
        Kc, Vc = Kc_o, Vc_o
    t = int(case.seq_lens[b]) - 1
    qg = _widen(case.q[b, g * G:(g + 1) * G])
    gates = _group_gates(case, qg, g, G, case.gates[b, g * G:(g + 1) * G])
    return nsa_query(qg, K, V, Kc, Vc, t, gates, p.l, p.d, p.l_sel, p.n_sel, p.n_local,
                     p.force_initial, p.w, override_idx=override_idx)


def prefill_rows(case, b: int, g: int, rows: Sequence[int], K=None, V=None, Kc=None, Vc=None,
                 override_idx=None):
    """Prefill outputs of sequence b, KV group g at the given query positions."""
    p = case.wl.params
    G = case.wl.num_q_heads // case.wl.num_kv_heads
    if K is None:
        K, V, Kc, Vc = compress_group(case, b, g)
    res = []
    for r, t in enumerate(rows):
        qg = _widen(case.q[b, t, g * G:(g + 1) * G])
        gates = _group_gates(case, qg, g, G, case.gates[b, t, g * G:(g + 1) * G])
        oi = None if override_idx is None else override_idx[r]
        res.append(nsa_query(qg, K, V, Kc, Vc, int(t), gates, p.l, p.d, p.l_sel, p.n_sel,
                             p.n_local, p.force_initial, p.w, override_idx=oi))
    return res


# --------------------------------------------------------------------------- compute budget

def keys_per_query_formula(N: int, stride: int, n: int, l_sel: int, w: int) -> float:
    """Keys read by one query: N/stride compressed + n*l' selected + w window.

    [LES "Compute budget": N/l + k*b + w per query; FLI "Сколько это экономит":
    t/16 compressed + 1024 selected + 512 window.]
    """
    return N / stride + n * l_sel + w


def keys_touched(t: int, l: int, d: int, l_sel: int, n: int, w: int) -> dict:
    """Keys each branch reads at query t by the definitions above (overlaps counted twice).

    Selected tokens assume every selected block is complete (t at a block end).
    """
    J = t // l_sel
    return dict(cmp=n_compressed(t + 1, l, d), slc=min(n, J + 1) * l_sel, win=min(w, t + 1))


def window_visible(i: np.ndarray, j: np.ndarray, w: int) -> np.ndarray:
    """Query i sees key j in the sliding window iff j <= i and i - j < w."""
    return (j <= i) & (i - j < w)
