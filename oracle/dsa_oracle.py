"""Plain float64 CPU oracle of a DeepSeek Sparse Attention (DSA) decode step.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the CPU
baseline leg of the benchmark may import this module; the library never does.
It shares no code with the HIP path.

Source: lesson 5.5/02 "Разреженное внимание — NSA и DSA" (ai.flicky.cc),
section "DSA: молниеносный индексатор" (the indexer equation, the selection of
2048 tokens per query, MLA in MQA mode over one shared 576-number latent per
token) and the practice spec of ``topk_mask`` / ``sparse_attention`` in
"Задание в браузере" (only keys j <= i; all of them when fewer than k;
1/sqrt(d) scale; row-max-subtracted softmax over the allowed keys).

One decode query at position t of one sequence:

  indexer     I[s] = sum_j w[j] * ReLU(qI[j] . kI[s]) for s <= t, with H^I small
              heads j; qI and kI are FP8 (OCP E4M3), w is float; no softmax.
  selection   the k tokens with the largest I[s], s <= t (ties to the lower s);
              every token when t + 1 <= k.  Returned ascending.
  attention   every one of the H query heads attends the selected tokens' latent
              vectors c[s] (d_qk numbers): logits scale * q[h] . c[s], softmax,
              output sum_s p * c[s][:d_v] (the values are the first d_v latent
              numbers).  scale defaults to 1/sqrt(d_qk).
"""
from __future__ import annotations

from typing import Optional

import numpy as np

from oracle.nsa_oracle import attend


def fp8_e4m3_to_float(bits: np.ndarray) -> np.ndarray:
    """OCP 8-bit floating point E4M3 bit patterns -> float64 (exact).

    One sign bit, four exponent bits with bias 7, three mantissa bits.  Exponent 0
    holds the subnormals m/8 * 2^-6; the pattern S.1111.111 is NaN (there is no
    infinity), so the largest finite magnitude is 1.75 * 2^8 = 448.
    """
    b = np.asarray(bits, dtype=np.uint8).astype(np.int64)
    sign = np.where(b & 0x80, -1.0, 1.0)
    e = (b >> 3) & 0xF
    m = b & 0x7
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    out = sign * mag
    return np.where((e == 15) & (m == 7), np.nan, out)


def indexer_scores(qI: np.ndarray, w: np.ndarray, kI: np.ndarray) -> np.ndarray:
    """I[s] = sum_j w[j] * ReLU(qI[j] . kI[s]).  qI [H^I, d_I], w [H^I], kI [n, d_I]."""
    dots = np.asarray(kI, dtype=np.float64) @ np.asarray(qI, dtype=np.float64).T   # [n, H^I]
    return np.maximum(dots, 0.0) @ np.asarray(w, dtype=np.float64)


def topk_tokens(I: np.ndarray, t: int, k: int) -> np.ndarray:
    """The k largest scores among positions 0..t (ties to the lower position), ascending."""
    n = t + 1
    if n <= k:
        return np.arange(n, dtype=np.int64)
    order = sorted(range(n), key=lambda s: (-I[s], s))
    return np.sort(np.array(order[:k], dtype=np.int64))


def dsa_decode_query(q: np.ndarray, qI: np.ndarray, w: np.ndarray, C: np.ndarray, kI: np.ndarray, t: int,
                     k: int, d_v: int, scale: Optional[float] = None, override_idx=None):
    """One DSA decode query.  q [H, d_qk] (float), qI [H^I, d_I] and kI [>= t+1, d_I]
    (float values of the FP8 inputs), w [H^I], C [>= t+1, d_qk] latent cache.

    Returns (out [H, d_v], idx, I) with I the indexer scores of positions 0..t.
    ``override_idx`` attends a given token set instead of the top-k."""
    I = indexer_scores(qI, w, kI[:t + 1])
    idx = np.asarray(override_idx, dtype=np.int64) if override_idx is not None else topk_tokens(I, t, k)
    d_qk = C.shape[1]
    s = 1.0 / np.sqrt(d_qk) if scale is None else scale
    Csel = np.asarray(C[idx], dtype=np.float64)
    out, _ = attend(q, Csel, Csel[:, :d_v], s)
    return out, idx, I


# --------------------------------------------------------------------------- batch driver

def _widen_bf16(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def decode_sequence(case, b: int, override_idx=None):
    """Oracle DSA decode step of sequence b of a DSA case (query at t = seq_lens[b] - 1)."""
    wl = case.wl
    t = int(case.seq_lens[b]) - 1
    q = _widen_bf16(case.q[b])
    C = _widen_bf16(case.c[b, :t + 1])
    qI = fp8_e4m3_to_float(case.q_idx[b])
    kI = fp8_e4m3_to_float(case.k_idx[b, :t + 1])
    w = np.asarray(case.w_idx[b], dtype=np.float64)
    return dsa_decode_query(q, qI, w, C, kI, t, wl.top_k, wl.d_v, override_idx=override_idx)
