"""Pins of the DSA oracle (CPU only): the FP8 decoder, the indexer score, the
token top-k and the sparse MQA attention, against closed forms, a worked
example, an independent FP8 implementation and brute force."""
import json
import os

import numpy as np
import pytest
import torch

from oracle import dsa_oracle as D

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_fp8_closed_forms():
    codes = np.array([0x38, 0x7E, 0x01, 0x08, 0x07, 0xB8, 0x00, 0x80, 0x40, 0x3C], dtype=np.uint8)
    want = [1.0, 448.0, 2.0 ** -9, 2.0 ** -6, 7 / 8 * 2.0 ** -6, -1.0, 0.0, -0.0, 2.0, 1.5]
    np.testing.assert_array_equal(D.fp8_e4m3_to_float(codes), want)
    assert np.isnan(D.fp8_e4m3_to_float(np.array([0x7F, 0xFF], np.uint8))).all()


def test_fp8_matches_an_independent_implementation():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = D.fp8_e4m3_to_float(codes)
    both_nan = np.isnan(ref) & np.isnan(got)
    assert np.array_equal(got[~both_nan], ref[~both_nan]) and both_nan.sum() == 2


def test_indexer_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "dsa_indexer_tiny.json")))
    I = D.indexer_scores(np.array(g["q_idx"], float), np.array(g["w_idx"], float), np.array(g["k_idx"], float))
    np.testing.assert_array_equal(I, g["scores"])
    np.testing.assert_array_equal(D.topk_tokens(I, 2, 2), g["top2_ascending"])
    np.testing.assert_array_equal(D.topk_tokens(I, 2, 1), g["top1"])   # tie between 0 and 2: lower wins


def test_indexer_properties():
    rng = np.random.default_rng(3)
    qI = rng.standard_normal((4, 8))
    w = rng.standard_normal(4)
    kI = rng.standard_normal((50, 8))
    I = D.indexer_scores(qI, w, kI)
    # one head, unit weight, query equal to a key: that key scores its squared norm
    np.testing.assert_allclose(D.indexer_scores(kI[7:8], np.ones(1), kI[7:8]), [np.dot(kI[7], kI[7])], rtol=1e-14)
    # a head whose dot is negative contributes nothing
    assert D.indexer_scores(-kI[3:4], np.ones(1), kI[3:4])[0] == 0.0
    # linear in w, invariant to a joint permutation of heads and weights
    np.testing.assert_allclose(D.indexer_scores(qI, 3 * w, kI), 3 * I, rtol=1e-13)
    perm = [2, 0, 3, 1]
    np.testing.assert_allclose(D.indexer_scores(qI[perm], w[perm], kI), I, rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("seed", range(6))
def test_topk_brute_force(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 40))
    I = np.round(rng.standard_normal(60), 1)      # coarse values: many ties
    t, k = n - 1, int(rng.integers(1, 12))
    S = D.topk_tokens(I, t, k)
    assert np.all(np.diff(S) > 0) and np.all(S <= t)           # ascending, never the future
    if t + 1 <= k:
        np.testing.assert_array_equal(S, np.arange(t + 1))
        return
    assert len(S) == k
    worst = min((I[s], -s) for s in S)
    for s in range(t + 1):
        if s not in S:
            assert (I[s], -s) < worst                          # nothing unselected ranks higher


def test_large_k_is_causal_attention():
    """The practice spec: k >= T gives plain causal attention over every past token."""
    rng = np.random.default_rng(4)
    T, H, dqk, dv = 9, 3, 12, 8
    q = rng.standard_normal((H, dqk))
    C = rng.standard_normal((T, dqk))
    qI, kI, w = rng.standard_normal((2, 4)), rng.standard_normal((T, 4)), rng.standard_normal(2)
    out, idx, _ = D.dsa_decode_query(q, qI, w, C, kI, T - 1, 64, dv)
    np.testing.assert_array_equal(idx, np.arange(T))
    z = q @ C.T / np.sqrt(dqk)
    p = np.exp(z - z.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    np.testing.assert_allclose(out, p @ C[:, :dv], rtol=1e-12, atol=1e-14)


def test_attention_reads_only_selected_tokens():
    """Changing an unselected token's latent leaves the output unchanged; the values are
    the first d_v latent numbers."""
    rng = np.random.default_rng(5)
    T, H, dqk, dv, k = 40, 2, 10, 6, 5
    q, C = rng.standard_normal((H, dqk)), rng.standard_normal((T, dqk))
    qI, kI, w = rng.standard_normal((3, 4)), rng.standard_normal((T, 4)), np.abs(rng.standard_normal(3))
    out, idx, _ = D.dsa_decode_query(q, qI, w, C, kI, T - 1, k, dv)
    other = [s for s in range(T) if s not in idx][0]
    C2 = C.copy()
    C2[other] += 100.0
    out2, idx2, _ = D.dsa_decode_query(q, qI, w, C2, kI, T - 1, k, dv)
    np.testing.assert_array_equal(idx, idx2)
    np.testing.assert_allclose(out, out2, rtol=1e-14)
    C3 = C.copy()
    C3[idx[0], dv:] += 1.0    # a non-value latent number moves the logits only
    out3, _, _ = D.dsa_decode_query(q, qI, w, C3, kI, T - 1, k, dv)
    assert not np.allclose(out3, out)


def test_read_fraction_from_the_pages():
    """At 128K tokens the main attention reads 2048 / 131072, about 1.6% of the keys."""
    assert abs(2048 / 131072 - 0.016) < 0.001
