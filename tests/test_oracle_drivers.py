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


# ---------------------------------------------------------------- layout pins of the drivers
#
# Each driver is run on a hand-built case whose rows are planted at the places
# the documented layouts name (the Case docstring: decode caches hold sequence b,
# KV head g, token x at row Hkv*cu[b] + g*cap_b + x; prefill k/v are
# [B, Hkv, T, D]; q and gates are [B, (T,) Hq, .]).  Every other row holds
# values that would change the result if read.  The expected outputs are closed
# forms: a query along one-hot direction r attends (up to e^-64) uniformly the
# tokens whose one-hot key is r, so each branch's output is the mean of their
# planted values.

def _onehot_bits(idx, n, scale):
    """bf16 bits of scale * e_idx (scale a power of two)."""
    x = np.zeros(n, np.float32)
    x[idx] = scale
    return I.bf16_bits(x)


def _residue(hq, g, b):
    return (hq + 5 * g + 3 * b) % 16


def _driver_params():
    # l = d = l' = 16 with mean-pool compression; every block selectable (n large)
    return I.NSAParams(l=16, d=16, l_sel=16, n_sel=64, n_local=2, force_initial=1, w=24)


def _mean_pool_weights(D, l):
    return I.bf16_bits(np.tile(np.eye(D, dtype=np.float32), (l, 1)) / np.float32(l))


def _expected_group(b, g, G, t, p, gates):
    """Closed-form NSA output of group g's heads at position t for the planted values
    V[x] = (b, g, x, 1), keys K[x] = e_{x mod 16}, queries 256 e_r."""
    out = []
    for h in range(G):
        r = _residue(g * G + h, g, b)
        win = [x for x in range(max(0, t - p.w + 1), t + 1) if x % 16 == r]
        slc = [x for x in range(t + 1) if x % 16 == r]
        nvis = O.n_compressed(t + 1, p.l, p.d)
        # compressed keys are all (1/16) * ones: uniform weights over the visible blocks,
        # whose mean values are (b, g, 16 i + 7.5, 1)
        o_cmp = np.array([b, g, 8.0 * (nvis - 1) + 7.5, 1.0]) if nvis else np.zeros(4)

        def mean_of(xs):
            return np.array([b, g, np.mean(xs), 1.0]) if xs else np.array([b, g, np.mean(range(t + 1)), 1.0])
        o = gates[h, 0] * o_cmp + gates[h, 1] * mean_of(slc) + gates[h, 2] * mean_of(win)
        out.append(o)
    return np.stack(out)


def _decode_case(gate_net=False):
    B, H, G, dk, dv = 3, 2, 16, 16, 4
    p = _driver_params()
    wl = I.Workload("driver_decode", "decode", B, H * G, H, dk, dv, 80, p, needles=0)
    caps = np.array([48, 80, 64], np.int64)
    lens = np.array([40, 77, 53], np.int32)
    cu = np.concatenate([[0], np.cumsum(caps)]).astype(np.int64)
    rng = np.random.default_rng(7)
    rows = H * int(cu[-1])
    k = I.bf16_bits(rng.standard_normal((rows, dk), dtype=np.float32) * 4)   # garbage unless planted
    v = I.bf16_bits(np.full((rows, dv), 1000.0, np.float32))
    for b in range(B):
        for g in range(H):
            for x in range(int(lens[b])):
                row = H * int(cu[b]) + g * int(caps[b]) + x
                k[row] = _onehot_bits(x % 16, dk, 1.0)
                v[row] = I.bf16_bits(np.array([b, g, x, 1.0], np.float32))
    q = np.zeros((B, H * G, dk), np.uint16)
    for b in range(B):
        for hq in range(H * G):
            q[b, hq] = _onehot_bits(_residue(hq, hq // G, b), dk, 256.0)
    gates = ((np.arange(B * H * G * 3, dtype=np.float32).reshape(B, H * G, 3) % 7) + 1) / np.float32(8)
    case = I.Case(wl=wl, seed=0, q=q, k=k, v=v, gates=gates,
                  w_k=_mean_pool_weights(dk, p.l), pe_k=np.zeros((p.l, dk), np.uint16),
                  w_v=_mean_pool_weights(dv, p.l), pe_v=np.zeros((p.l, dv), np.uint16),
                  seq_lens=lens, cu_seqlens=cu)
    if gate_net:
        # hand-set gate network: head hq's window gate reads query component r(hq)
        # with weight m/256, so z_win = m = (hq % 5) - 2; cmp / slc gates from the bias only
        w_gate = np.zeros((H * G, 3, dk), np.float32)
        for hq in range(H * G):
            w_gate[hq, 2, _residue(hq, hq // G, 0)] = ((hq % 5) - 2) / 256.0
        case.w_gate = I.bf16_bits(w_gate)
        case.b_gate = np.tile(np.array([[-1.0, 0.5, 0.25]], np.float32), (H * G, 1))
        case.gate_net = True
    return case


def test_decode_driver_reads_the_documented_rows_and_heads():
    case = _decode_case()
    p, G = case.p, 16
    for b in range(3):
        for g in range(2):
            r = O.decode_group(case, b, g)
            t = int(case.seq_lens[b]) - 1
            want = _expected_group(b, g, G, t, p, case.gates[b, g * G:(g + 1) * G].astype(np.float64))
            np.testing.assert_allclose(r.out, want, rtol=1e-12, atol=1e-12)
            assert r.idx == list(range(t // p.l_sel + 1))


def test_decode_driver_gate_network_reads_its_heads_weights():
    case = _decode_case(gate_net=True)
    p, G = case.p, 16
    sig = lambda z: 1.0 / (1.0 + np.exp(-z))
    for b, g in ((0, 1), (2, 0)):
        t = int(case.seq_lens[b]) - 1
        gates = np.zeros((G, 3))
        for h in range(G):
            hq = g * G + h
            # the window weight sits on component r(hq) computed for b = 0; it meets the
            # query's 256 only when the query's residue (which depends on b) is the same
            hit = _residue(hq, g, b) == _residue(hq, g, 0)
            gates[h] = sig(np.array([-1.0, 0.5, 0.25 + (((hq % 5) - 2) if hit else 0.0)]))
        r = O.decode_group(case, b, g)
        np.testing.assert_allclose(r.out, _expected_group(b, g, G, t, p, gates), rtol=1e-12, atol=1e-12)


def test_prefill_driver_reads_the_documented_rows_and_heads():
    B, H, G, dk, dv, T = 2, 2, 16, 16, 4, 70
    p = _driver_params()
    wl = I.Workload("driver_prefill", "prefill", B, H * G, H, dk, dv, T, p, needles=0)
    k = np.zeros((B, H, T, dk), np.uint16)
    v = np.zeros((B, H, T, dv), np.uint16)
    for b in range(B):
        for g in range(H):
            for x in range(T):
                k[b, g, x] = _onehot_bits(x % 16, dk, 1.0)
                v[b, g, x] = I.bf16_bits(np.array([b, g, x, 1.0], np.float32))
    q = np.zeros((B, T, H * G, dk), np.uint16)
    for b in range(B):
        for t in range(T):
            for hq in range(H * G):
                q[b, t, hq] = _onehot_bits((_residue(hq, hq // G, b) + t) % 16, dk, 256.0)
    gates = (((np.arange(B * T * H * G * 3, dtype=np.float32).reshape(B, T, H * G, 3) % 11) + 1) / np.float32(16))
    case = I.Case(wl=wl, seed=0, q=q, k=k, v=v, gates=gates,
                  w_k=_mean_pool_weights(dk, p.l), pe_k=np.zeros((p.l, dk), np.uint16),
                  w_v=_mean_pool_weights(dv, p.l), pe_v=np.zeros((p.l, dv), np.uint16))
    rows = [0, 15, 16, 37, 69]
    for b, g in ((1, 1), (0, 1), (1, 0)):
        res = O.prefill_rows(case, b, g, rows)
        for t, r in zip(rows, res):
            # the query at t points along residue r(hq) + t: shift the planted residue
            want = []
            for h in range(G):
                hq = g * G + h
                rr = (_residue(hq, g, b) + t) % 16
                win = [x for x in range(max(0, t - p.w + 1), t + 1) if x % 16 == rr]
                slc = [x for x in range(t + 1) if x % 16 == rr]
                nvis = O.n_compressed(t + 1, p.l, p.d)
                o_cmp = np.array([b, g, 8.0 * (nvis - 1) + 7.5, 1.0]) if nvis else np.zeros(4)
                full = np.array([b, g, np.mean(range(t + 1)), 1.0])
                o_slc = np.array([b, g, np.mean(slc), 1.0]) if slc else full
                o_win = np.array([b, g, np.mean(win), 1.0]) if win else full
                gt = case.gates[b, t, hq].astype(np.float64)
                want.append(gt[0] * o_cmp + gt[1] * o_slc + gt[2] * o_win)
            np.testing.assert_allclose(r.out, np.stack(want), rtol=1e-12, atol=1e-12)


def test_compress_group_reads_the_documented_rows():
    """compress_group of a decode case compresses exactly sequence b, head g's rows:
    with mean-pool weights block i's value is (b, g, 16 i + 7.5, 1)."""
    case = _decode_case()
    for b in range(3):
        for g in range(2):
            _, V, _, Vc = O.compress_group(case, b, g)
            L = int(case.seq_lens[b])
            assert V.shape[0] == L
            nc = O.n_compressed(L, 16, 16)
            want = np.array([[b, g, 16 * i + 7.5, 1.0] for i in range(nc)])
            np.testing.assert_array_equal(Vc, want)


def test_dsa_driver_reads_the_documented_rows():
    """dsa_oracle.decode_sequence on a hand-built case: sequence b's planted indexer
    keys (FP8 2.0 along the query's first component) win the top-k; planted keys past
    the sequence's length and in other sequences' rows must not; each head then
    attends the planted token whose latent carries its one-hot logit direction."""
    from oracle import dsa_oracle as D
    B, Hh, dqk, dv, HI, DI, cap, topk = 3, 4, 8, 4, 2, 4, 40, 3
    wl = I.DsaWorkload("driver_dsa", B, Hh, dqk, dv, HI, DI, topk, cap, needles=0)
    lens = np.array([30, 40, 17], np.int32)
    planted = {0: [4, 9, 26], 1: [0, 21, 38], 2: [8, 13, 2]}
    q_idx = np.zeros((B, HI, DI), np.uint8)
    q_idx[:, 0, 0] = 0x38                                      # 1.0
    k_idx = np.zeros((B, cap, DI), np.uint8)
    c = np.zeros((B, cap, dqk), np.float32)
    for b in range(B):
        c[b, :, :4] = np.stack([np.full(cap, b), np.arange(cap), np.zeros(cap), np.ones(cap)], axis=1)
        for s in planted[b]:
            k_idx[b, s, 0] = 0x40                              # 2.0
            c[b, s, 4 + s % 4] = 1.0
        k_idx[b, lens[b]:, 0] = 0x48                           # 4.0 beyond the length: never visible
    w_idx = np.tile(np.array([[1.0, 0.0]], np.float32), (B, 1))
    q = np.zeros((B, Hh, dqk), np.float32)
    for b in range(B):
        for h in range(Hh):
            q[b, h, 4 + (h + b) % 4] = 256.0
    case = I.DsaCase(wl=wl, seed=0, q=I.bf16_bits(q), c=I.bf16_bits(c), q_idx=q_idx, k_idx=k_idx,
                     w_idx=w_idx, seq_lens=lens)
    for b in range(B):
        out, idx, scores = D.decode_sequence(case, b)
        assert list(idx) == sorted(planted[b])
        assert scores.shape == (int(lens[b]),)
        for h in range(Hh):
            hits = [s for s in planted[b] if s % 4 == (h + b) % 4]
            want = np.array([b, np.mean(hits if hits else planted[b]), 0.0, 1.0])
            np.testing.assert_allclose(out[h], want, rtol=1e-12, atol=1e-12)
