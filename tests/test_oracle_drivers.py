"""The oracle's batch drivers on seeded workloads (CPU only)."""
import numpy as np

import nsa_inputs as I
from oracle import nsa_oracle as O


def test_generator_is_seeded():
    wl = I.workload("decode_64k_b8", seq_len=1024, batch=2)
    a, b = I.generate(wl, 3), I.generate(wl, 3)
    for name in ("q", "k", "v", "w_k", "pe_v"):
        np.testing.assert_array_equal(getattr(a, name), getattr(b, name))
    np.testing.assert_array_equal(a.gates, b.gates)
    c = I.generate(wl, 4)
    assert not np.array_equal(a.k, c.k)


def test_tiny_prefill_runs_and_respects_invariants():
    case = I.generate(I.workload("tiny_prefill_512"), 0, keep_fp32=True)
    p = case.p
    res = O.prefill_rows(case, 0, 0, range(512))
    for t, r in enumerate(res):
        J = t // p.l_sel
        assert len(r.idx) == min(p.n_sel, J + 1)
        assert 0 in r.idx and J in r.idx and max(r.idx) <= J
        if O.n_compressed(t + 1, p.l, p.d):
            assert abs(r.scores.sum() - 4) < 1e-9
    out = np.stack([r.out for r in res])
    assert np.isfinite(out).all()


def test_tiny_prefill_fp32_vs_bf16_inputs():
    """Oracle-only: the same workload on unrounded fp32 inputs stays close to the bf16 run."""
    case = I.generate(I.workload("tiny_prefill_512"), 0, keep_fp32=True)
    p = case.p
    f = case.fp32
    K, V = f["k"][0, 0].astype(np.float64), f["v"][0, 0].astype(np.float64)
    Kc = O.compress(K, f["w_k"].astype(np.float64), f["pe_k"].astype(np.float64), p.l, p.d, round_bf16=False)
    Vc = O.compress(V, f["w_v"].astype(np.float64), f["pe_v"].astype(np.float64), p.l, p.d, round_bf16=False)
    rows = range(0, 512, 7)
    r16 = O.prefill_rows(case, 0, 0, rows)
    diffs = []
    for r, t in zip(r16, rows):
        r32 = O.nsa_query(f["q"][0, t].astype(np.float64), K, V, Kc, Vc, t, case.gates[0, t].astype(np.float64),
                          p.l, p.d, p.l_sel, p.n_sel, p.n_local, p.force_initial, p.w,
                          override_idx=r.idx)
        diffs.append(np.abs(r32.out - r.out).max())
    assert max(diffs) < 5e-2


def test_small_decode_batch():
    wl = I.workload("decode_64k_b8", seq_len=3000, batch=2)
    case = I.generate(wl, 1)
    for b in range(2):
        for g in range(wl.num_kv_heads):
            r = O.decode_group(case, b, g)
            assert len(r.idx) == wl.params.n_sel
            assert r.out.shape == (16, wl.d_v)


def test_ragged_decode_lengths():
    wl = I.workload("decode_ragged_16", batch=3, seq_len=5000, ragged_min=100)
    case = I.generate(wl, 2)
    assert case.seq_lens.min() >= 100 and case.seq_lens.max() <= 5000
    assert case.k.shape[0] == wl.num_kv_heads * int(case.seq_lens.sum())
    r = O.decode_group(case, 2, 3)
    assert np.isfinite(r.out).all()
