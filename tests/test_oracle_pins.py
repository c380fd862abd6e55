"""Pins of the CPU oracle against what the pages and the mathematics fix.

None of these re-types the oracle's formulas: each compares it with a library
routine (torch's scaled-dot-product attention in float64), a closed form, a
brute-force search, an invariant, or a value printed on the pages
(tests/golden/, each file citing its source).
"""
import itertools
import json
import os

import numpy as np
import pytest
import torch

from oracle import nsa_oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _causal_sdpa(q, K, V):
    """Causal attention by torch's SDPA in float64: q [T,H,dk], K [T,dk], V [T,dv] -> [T,H,dv]."""
    qt = torch.tensor(q).permute(1, 0, 2)                       # [H,T,dk]
    H = qt.shape[0]
    Kt = torch.tensor(K)[None].expand(H, -1, -1).contiguous()
    Vt = torch.tensor(V)[None].expand(H, -1, -1).contiguous()
    o = torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt, is_causal=True)
    return o.permute(1, 0, 2).numpy()


def _rand(rng, *shape):
    # bf16-exact values so the compressed-cache rounding is an identity where it must be
    return O.round_to_bf16(rng.standard_normal(shape))


def _run_all(q, K, V, Kc, Vc, gates, **p):
    T = q.shape[0]
    return [O.nsa_query(q[t], K, V, Kc, Vc, t, gates, **p) for t in range(T)]


# ---------------------------------------------------------------- reductions to causal attention

@pytest.mark.parametrize("T,l_sel", [(40, 8), (37, 16)])
def test_window_only_is_causal(T, l_sel):
    rng = np.random.default_rng(1)
    G, dk, dv = 3, 8, 5
    q, K, V = rng.standard_normal((T, G, dk)), rng.standard_normal((T, dk)), rng.standard_normal((T, dv))
    gates = np.tile([0.0, 0.0, 1.0], (G, 1))
    Kc = O.compress(K, rng.standard_normal((4 * dk, dk)) * 0.1, np.zeros((4, dk)), 4, 2)
    Vc = O.compress(V, rng.standard_normal((4 * dv, dv)) * 0.1, np.zeros((4, dv)), 4, 2)
    res = _run_all(q, K, V, Kc, Vc, gates, l=4, d=2, l_sel=l_sel, n=2, n_local=1, force_initial=1, w=T + 5)
    ref = _causal_sdpa(q, K, V)
    got = np.stack([r.out for r in res])
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("T,l_sel", [(40, 8), (45, 16)])
def test_select_all_is_causal(T, l_sel):
    rng = np.random.default_rng(2)
    G, dk, dv, l, d = 2, 8, 6, 4, 2
    q, K, V = rng.standard_normal((T, G, dk)), rng.standard_normal((T, dk)), rng.standard_normal((T, dv))
    W = _rand(rng, l * dk, dk) * 0.1
    Kc = O.compress(K, W, np.zeros((l, dk)), l, d)
    Vc = O.compress(V, _rand(rng, l * dv, dv) * 0.1, np.zeros((l, dv)), l, d)
    gates = np.tile([0.0, 1.0, 0.0], (G, 1))
    n = -(-T // l_sel)
    res = _run_all(q, K, V, Kc, Vc, gates, l=l, d=d, l_sel=l_sel, n=n, n_local=1, force_initial=1, w=3)
    np.testing.assert_allclose(np.stack([r.out for r in res]), _causal_sdpa(q, K, V), rtol=1e-12, atol=1e-12)
    for t, r in enumerate(res):
        assert r.idx == list(range(t // l_sel + 1))


def test_identity_compression_is_causal():
    """l = d = 1, W = I, PE = 0: every token is its own compressed block."""
    rng = np.random.default_rng(3)
    T, G, dk = 33, 4, 8
    q, K, V = rng.standard_normal((T, G, dk)), _rand(rng, T, dk), _rand(rng, T, dk)
    Kc = O.compress(K, np.eye(dk), np.zeros((1, dk)), 1, 1)
    Vc = O.compress(V, np.eye(dk), np.zeros((1, dk)), 1, 1)
    np.testing.assert_array_equal(Kc, K)
    gates = np.tile([1.0, 0.0, 0.0], (G, 1))
    res = _run_all(q, K, V, Kc, Vc, gates, l=1, d=1, l_sel=4, n=2, n_local=1, force_initial=1, w=4)
    np.testing.assert_allclose(np.stack([r.out for r in res]), _causal_sdpa(q, K, V), rtol=1e-12, atol=1e-12)


def test_compression_visibility_and_flatten_order():
    """l=2, d=1, W picks channel perm(c) of the block's LAST token: kc_i = P K[i+1] + PE[1] P.

    So block i becomes visible exactly when token i+1 arrives, and the compressed
    branch equals causal attention over keys 1..t of the permuted keys.
    """
    rng = np.random.default_rng(4)
    T, G, dk, l, d = 30, 2, 6, 2, 1
    q, K, V = rng.standard_normal((T, G, dk)), _rand(rng, T, dk), _rand(rng, T, dk)
    perm = rng.permutation(dk)
    W = np.zeros((l * dk, dk))
    for c2 in range(dk):
        W[(l - 1) * dk + perm[c2], c2] = 1.0      # token-major flatten: index j*dk + c
    Kc = O.compress(K, W, np.zeros((l, dk)), l, d)
    np.testing.assert_array_equal(Kc, K[1:][:, perm])
    Vc = O.compress(V, W, np.zeros((l, dk)), l, d)
    gates = np.tile([1.0, 0.0, 0.0], (G, 1))
    res = _run_all(q, K, V, Kc, Vc, gates, l=l, d=d, l_sel=4, n=2, n_local=1, force_initial=1, w=4)
    assert np.all(res[0].o_cmp == 0.0)            # no complete block at t = 0
    ref = _causal_sdpa(q[1:], K[1:][:, perm], V[1:][:, perm])
    np.testing.assert_allclose(np.stack([r.out for r in res[1:]]), ref, rtol=1e-12, atol=1e-12)


def test_position_embedding_adds_per_token():
    """W = I on the last token: kc_i = K[i*d+l-1] + PE[l-1] (before bf16 rounding)."""
    rng = np.random.default_rng(5)
    L, D, l, d = 50, 4, 4, 2
    K = rng.standard_normal((L, D))
    PE = rng.standard_normal((l, D))
    W = np.zeros((l * D, D))
    W[(l - 1) * D:, :] = np.eye(D)
    kc = O.compress(K, W, PE, l, d, round_bf16=False)
    nc = (L - l) // d + 1
    np.testing.assert_allclose(kc, K[np.arange(nc) * d + l - 1] + PE[l - 1], rtol=0, atol=1e-14)


def test_mean_pool_compressor_is_block_mean():
    """W = (1/l)[I; ...; I], d = l: the lesson's mean-pool compressor on complete blocks."""
    rng = np.random.default_rng(6)
    L, D, l = 70, 5, 8
    K = rng.standard_normal((L, D))
    W = np.tile(np.eye(D), (l, 1)) / l
    kc = O.compress(K, W, np.zeros((l, D)), l, l, round_bf16=False)
    nb = L // l
    np.testing.assert_allclose(kc, K[:nb * l].reshape(nb, l, D).mean(axis=1), rtol=1e-13, atol=1e-14)


def test_nc_closed_form():
    assert O.n_compressed(65536, 32, 16) == 4095
    assert O.n_compressed(131072, 32, 16) == 8191
    assert O.n_compressed(32768, 32, 16) == 2047
    assert O.n_compressed(31, 32, 16) == 0 and O.n_compressed(32, 32, 16) == 1


@pytest.mark.parametrize("l,d", [(32, 16), (8, 8), (6, 2)])
def test_one_block_completes_every_d_tokens(l, d):
    """Growing a sequence one token at a time adds exactly one compressed block at
    t = i*d + l - 1 (the block ending at the new token) and none otherwise; every
    earlier block is unchanged (a block reads only its own l tokens).  This is the
    rule the streaming append follows, checked against the batch definition."""
    rng = np.random.default_rng(7)
    D = 4
    K = rng.standard_normal((120, D))
    W = rng.standard_normal((l * D, D))
    PE = rng.standard_normal((l, D))
    prev = O.compress(K[:0], W, PE, l, d, round_bf16=False)
    for L in range(1, 121):
        cur = O.compress(K[:L], W, PE, l, d, round_bf16=False)
        t = L - 1
        due = t >= l - 1 and (t - (l - 1)) % d == 0
        assert cur.shape[0] == prev.shape[0] + (1 if due else 0)
        np.testing.assert_allclose(cur[:prev.shape[0]], prev, rtol=1e-12, atol=1e-12)  # BLAS blocking may differ
        if due:
            i = (t - (l - 1)) // d
            assert cur.shape[0] == i + 1
            np.testing.assert_allclose(cur[i], ((K[t - l + 1:t + 1] + PE).reshape(-1)) @ W, rtol=1e-12)
        prev = cur


# ---------------------------------------------------------------- gate network

def test_gate_network_closed_forms():
    """sigmoid(0) = 1/2; a one-hot query picks weight column k of its own head
    (a transposed or head-mixed operand fails); sigmoid(-z) = 1 - sigmoid(z);
    saturation without overflow."""
    rng = np.random.default_rng(11)
    G, dk = 3, 8
    W = rng.standard_normal((G, 3, dk))
    b = rng.standard_normal((G, 3))
    np.testing.assert_array_equal(O.gate_network(np.zeros((G, dk)), W, None), np.full((G, 3), 0.5))
    for k in (0, 5):
        q = np.zeros((G, dk))
        q[:, k] = 1.0
        want = 1.0 / (1.0 + np.exp(-(W[:, :, k] + b)))
        np.testing.assert_allclose(O.gate_network(q, W, b), want, rtol=1e-15)
    q = rng.standard_normal((G, dk))
    np.testing.assert_allclose(O.gate_network(q, -W, -b), 1.0 - O.gate_network(q, W, b), rtol=1e-13, atol=1e-15)
    with np.errstate(over="ignore"):
        sat = O.gate_network(np.full((G, dk), 100.0), np.sign(W) * 10.0, None)
    assert np.all((sat == 0.0) | (sat == 1.0) | ((sat > 0) & (sat < 1)))
    # head independence: changing head 1's weights changes only head 1's gates
    W2 = W.copy()
    W2[1] += 1.0
    d = O.gate_network(q, W2, b) - O.gate_network(q, W, b)
    assert np.all(d[[0, 2]] == 0.0) and np.all(d[1] != 0.0)


# ---------------------------------------------------------------- gating

def test_gates_isolate_and_are_linear():
    rng = np.random.default_rng(7)
    T, G, dk, dv, l, d, l_sel = 90, 4, 8, 8, 8, 4, 16
    q, K, V = rng.standard_normal((T, G, dk)), _rand(rng, T, dk), _rand(rng, T, dv)
    Kc = O.compress(K, _rand(rng, l * dk, dk) * 0.2, _rand(rng, l, dk) * 0.02, l, d)
    Vc = O.compress(V, _rand(rng, l * dv, dv) * 0.2, _rand(rng, l, dv) * 0.02, l, d)
    p = dict(l=l, d=d, l_sel=l_sel, n=3, n_local=1, force_initial=1, w=20)
    gates = rng.uniform(0, 1, size=(G, 3))
    for t in (5, 31, 64, 89):
        r = O.nsa_query(q[t], K, V, Kc, Vc, t, gates, **p)
        one = [O.nsa_query(q[t], K, V, Kc, Vc, t, np.tile(np.eye(3)[b], (G, 1)), **p).out for b in range(3)]
        np.testing.assert_allclose(one[0], r.o_cmp, rtol=0, atol=0)
        np.testing.assert_allclose(one[1], r.o_slc, rtol=0, atol=0)
        np.testing.assert_allclose(one[2], r.o_win, rtol=0, atol=0)
        lin = sum(gates[:, b:b + 1] * one[b] for b in range(3))
        np.testing.assert_allclose(r.out, lin, rtol=1e-14, atol=1e-14)
        # gates need not sum to one: doubling every gate doubles the output
        r2 = O.nsa_query(q[t], K, V, Kc, Vc, t, 2 * gates, **p)
        np.testing.assert_allclose(r2.out, 2 * r.out, rtol=1e-14, atol=1e-14)


# ---------------------------------------------------------------- fold

@pytest.mark.parametrize("l,d,l_sel", [(32, 16, 64), (32, 16, 32), (8, 4, 16), (4, 4, 4)])
def test_fold_conserves_mass(l, d, l_sel):
    rng = np.random.default_rng(8)
    T, G, dk = 300, 3, 8
    q, K, V = rng.standard_normal((T, G, dk)), _rand(rng, T, dk), _rand(rng, T, dk)
    Kc = O.compress(K, _rand(rng, l * dk, dk) * 0.3, np.zeros((l, dk)), l, d)
    for t in (l - 1, l + d, 100, 299):
        r = O.nsa_query(q[t], K, V, Kc, Kc, t, np.ones((G, 3)), l=l, d=d, l_sel=l_sel, n=2,
                        n_local=1, force_initial=1, w=16)
        assert abs(r.scores.sum() - G) < 1e-12
        assert np.all(r.scores >= 0)


def test_fold_weights_closed_form():
    # l = d = l': identity
    om = O.fold_weights(10, 8, 8, 8, 10)
    np.testing.assert_array_equal(om, np.eye(10))
    # l=32, d=16, l'=64: blocks 4j..4j+2 lie in j; block 4j+3 is split half/half
    om = O.fold_weights(16, 32, 16, 64, 5)
    for i in range(16):
        j = i // 4
        if i % 4 == 3:
            assert om[i, j] == 0.5 and om[i, j + 1] == 0.5
        else:
            assert om[i, j] == 1.0
        assert om[i].sum() == 1.0
    # l=32, d=16, l'=32: even blocks whole, odd blocks split
    om = O.fold_weights(8, 32, 16, 32, 5)
    for i in range(8):
        if i % 2 == 0:
            assert om[i, i // 2] == 1.0
        else:
            assert om[i, i // 2] == 0.5 and om[i, i // 2 + 1] == 0.5


def test_single_head_ranking_matches_raw_logits():
    """With one head and l = d = l', ranking by probability equals ranking by q.kc."""
    rng = np.random.default_rng(9)
    T, dk, l = 256, 16, 16
    q, K, V = rng.standard_normal((1, dk)), _rand(rng, T, dk), _rand(rng, T, dk)
    W = np.tile(np.eye(dk), (l, 1)) / l
    Kc = O.compress(K, W, np.zeros((l, dk)), l, l)
    r = O.nsa_query(q, K, V, Kc, Kc, T - 1, np.ones((1, 3)), l=l, d=l, l_sel=l, n=5,
                    n_local=0, force_initial=0, w=8)
    raw = Kc @ q[0]
    assert r.idx == sorted(np.argsort(-raw, kind="stable")[:5].tolist())


# ---------------------------------------------------------------- top-n

def _forced_by_definition(J, n_local, force_initial):
    """The always-taken blocks written out from the selection paragraph, without the
    oracle: the initial block (when forced) and the n_local blocks ending at the
    query's own block J, clipped at 0."""
    F = set(range(max(0, J - n_local + 1), J + 1))
    if force_initial:
        F.add(0)
    return F


def _brute_topn(S, J, n, n_local, force_initial):
    F = _forced_by_definition(J, n_local, force_initial)
    rest = [j for j in range(J + 1) if j not in F]
    best, best_key = None, None
    for comb in itertools.combinations(rest, n - len(F)):
        # maximise the summed score; among equal sums prefer the lexicographically
        # smallest list of indices (ties to the lower block)
        key = (sum(S[j] for j in comb), tuple(-j for j in comb))
        if best_key is None or key > best_key:
            best, best_key = comb, key
    return sorted(F | set(best))


@pytest.mark.parametrize("seed", range(25))
def test_topn_brute_force(seed):
    rng = np.random.default_rng(100 + seed)
    J = int(rng.integers(0, 11))
    n = int(rng.integers(1, 7))
    n_local = int(rng.integers(0, min(n, 3) + 1))
    force_initial = int(rng.integers(0, 2)) if n > n_local else 0
    S = rng.uniform(0, 1, size=J + 1)
    got = O.select_blocks(S, J, n, n_local, force_initial)
    if J + 1 <= n:
        assert got == list(range(J + 1))
        return
    assert got == _brute_topn(S, J, n, n_local, force_initial)
    assert len(got) == n and max(got) <= J and got == sorted(got)


def test_forced_blocks_hand_examples():
    """Worked by hand from the selection paragraph ("always the initial block and two
    local ones"): at J = 10 the local blocks are 9 and 10, so with n = 5 two routed
    picks remain and go to the two best other blocks (3 and 7 here)."""
    S = np.array([0.0, 0.1, 0.2, 0.9, 0.1, 0.3, 0.2, 0.8, 0.85, 0.05, 0.95])
    # the routed picks are the two best of blocks 1..8: 3 (0.9) and 8 (0.85); 10 (0.95) is local anyway
    assert O.select_blocks(S, 10, 5, 2, 1) == [0, 3, 8, 9, 10]
    S2 = np.array([0.0, 0.1, 0.2, 0.9, 0.1, 0.3, 0.2, 0.8, 0.05, 0.97, 0.99])
    assert O.select_blocks(S2, 10, 5, 2, 1) == [0, 3, 7, 9, 10]
    assert O.forced_blocks(10, 2, 1) == [0, 9, 10]
    assert O.forced_blocks(1, 2, 1) == [0, 1]            # J - 1 = 0 merges with the initial block
    assert O.forced_blocks(0, 2, 1) == [0]
    assert O.forced_blocks(10, 2, 0) == [9, 10]
    assert O.forced_blocks(10, 1, 1) == [0, 10]
    # n = 4 at J = 10 with block 0 and two local blocks forced: one routed pick
    assert O.select_blocks(S2, 10, 4, 2, 1) == [0, 3, 9, 10]
    # J + 1 <= n: every block, forced or not
    assert O.select_blocks(S2[:4], 3, 4, 2, 1) == [0, 1, 2, 3]


def test_topn_ties_go_to_lower_index():
    S = np.array([0.5, 0.2, 0.2, 0.2, 0.9, 0.2, 0.1])
    # J = 6, n = 4, forced {0, 6}: two routed slots; 0.9 at 4 then the lowest-index 0.2
    assert O.select_blocks(S, 6, 4, 1, 1) == [0, 1, 4, 6]
    assert O.select_blocks(np.zeros(9), 8, 3, 0, 0) == [0, 1, 2]
    assert O.select_blocks(np.ones(9), 8, 3, 1, 1) == [0, 1, 8]


def test_topn_masks_never_select_future():
    """Row-wise invariants of a top-k mask: at most k entries per row, none above the diagonal."""
    rng = np.random.default_rng(11)
    T = 12
    scores = rng.standard_normal((T, T))
    for i in range(T):
        got = O.select_blocks(scores[i, :i + 1], i, 2, 0, 0)
        assert len(got) <= 2 and all(j <= i for j in got)


# ---------------------------------------------------------------- compute budget

def test_budget_formula_matches_pages():
    gold = json.load(open(os.path.join(GOLD, "savings.json")))
    for row in gold["budget"]:
        k = O.keys_per_query_formula(row["N"], row["stride"], row["n"], row["l_sel"], row["w"])
        assert k == row["keys"]
        if "ratio" in row:
            # the lesson truncates at the printed precision (1024/288 = 3.56 is shown as 3.5)
            dec = 0 if float(row["ratio"]).is_integer() else 1
            assert np.floor(row["full"] / k * 10 ** dec) / 10 ** dec == row["ratio"]
    tp = gold["table_params"]
    for row in gold["table"]:
        k = O.keys_per_query_formula(row["N"], tp["stride"], tp["n"], tp["l_sel"], tp["w"])
        assert k == row["keys_approx"]
        assert round(row["N"] / k, 1) == row["ratio"]


def test_counted_keys_agree_with_formula():
    """The branch definitions touch Nc(t+1) + n*l' + w keys, within one block of N/d."""
    for N in (8192, 16384, 32768, 65536):
        c = O.keys_touched(N - 1, 32, 16, 64, 16, 512)
        assert c["slc"] == 1024 and c["win"] == 512
        assert abs(c["cmp"] - N / 16) <= 32 / 16


# ---------------------------------------------------------------- masks and the needle demo

def test_window_mask_example():
    rows = [l for l in open(os.path.join(GOLD, "window_mask_T4_w2.txt")) if not l.startswith("#")]
    want = np.array([[int(x) for x in r.split()] for r in rows], dtype=bool)
    i, j = np.arange(4)[:, None], np.arange(4)[None, :]
    np.testing.assert_array_equal(O.window_visible(i, j, 2), want)


def test_window_with_sink_pair_fraction():
    g = json.load(open(os.path.join(GOLD, "flex_mask_fraction.json")))
    T = g["T"]
    i, j = np.arange(T)[:, None], np.arange(T)[None, :]
    keep = O.window_visible(i, j, g["window"]) | ((j < g["sink"]) & (j <= i))
    frac = keep.sum() / (j <= i).sum()
    assert round(float(frac), 3) == g["fraction"]


def test_window_branch_key_set():
    """The window branch of the oracle attends exactly the keys the mask allows."""
    rng = np.random.default_rng(12)
    T, dk, w = 20, 4, 6
    K, V = rng.standard_normal((T, dk)), np.eye(T)[:, :T]       # one-hot values reveal weights
    q = np.zeros((1, dk))                                       # uniform weights
    for t in range(T):
        nc = O.n_compressed(T, 4, 2)
        r = O.nsa_query(q, K, V, np.zeros((nc, dk)), np.zeros((nc, T)), t, np.ones((1, 3)),
                        l=4, d=2, l_sel=4, n=1, n_local=1, force_initial=0, w=w)
        want = O.window_visible(np.array(t), np.arange(T), w).astype(float)
        np.testing.assert_allclose(r.o_win[0], want / want.sum(), rtol=0, atol=1e-15)


def _needle_setup():
    rng = np.random.default_rng(0)
    T, dh = 8192, 64
    q = rng.normal(size=dh)
    K = rng.normal(size=(T, dh))
    V = rng.normal(size=(T, dh))
    nd = np.arange(3000, 3016)
    K[nd] = 8.0 * np.sqrt(dh) * q / np.dot(q, q) + 0.1 * rng.normal(size=(nd.size, dh))
    V[nd] = 3.0
    rand256 = np.sort(rng.choice(T, 256, replace=False))
    return q, K, V, nd, rand256


def test_needle_demo_values():
    gold = json.load(open(os.path.join(GOLD, "needle_demo.json")))
    q, K, V, nd, rand256 = _needle_setup()
    T, dh = K.shape
    s = 1.0 / np.sqrt(dh)
    full, p_full = O.attend(q[None], K, V, s)
    assert round(float(p_full[0, nd].sum()), 2) == gold["needle_weight_full"]

    def cos(a, b):
        return float(a @ b / np.linalg.norm(a) / np.linalg.norm(b))

    win = np.arange(T - 512, T)
    o_w, _ = O.attend(q[None], K[win], V[win], s)
    assert round(cos(o_w[0], full[0]), 3) == gold["window_512"]["cos"]
    o_r, _ = O.attend(q[None], K[rand256], V[rand256], s)
    assert round(cos(o_r[0], full[0]), 3) == gold["random_256"]["cos"]
    # block selection through the oracle: mean-pool compression (l = d = l' = 64),
    # compressed-branch probabilities as scores, plain top-16 (no forced blocks)
    B = 64
    Wmean = np.tile(np.eye(dh), (B, 1)) / B
    Kc = O.compress(K, Wmean, np.zeros((B, dh)), B, B, round_bf16=False)
    r = O.nsa_query(q[None], K, V, Kc, Kc, T - 1, np.ones((1, 3)), l=B, d=B, l_sel=B, n=16,
                    n_local=0, force_initial=0, w=512)
    sel = np.concatenate([np.arange(j * B, (j + 1) * B) for j in r.idx])
    union = np.union1d(sel, win)
    gw = gold["top16_blocks_plus_window"]
    assert union.size == gw["keys"]
    assert round(union.size / T, 3) == gw["frac"]
    o_u, _ = O.attend(q[None], K[union], V[union], s)
    assert round(cos(o_u[0], full[0]), 3) == gw["cos"]
    assert (3000 // B) in r.idx and (3015 // B) in r.idx


# ---------------------------------------------------------------- primitives

def test_attend_special_cases():
    rng = np.random.default_rng(13)
    V = rng.standard_normal((7, 3))
    o, p = O.attend(np.zeros((2, 4)), rng.standard_normal((7, 4)), V, 0.5)
    np.testing.assert_allclose(o, np.tile(V.mean(axis=0), (2, 1)), rtol=1e-14, atol=1e-15)
    o, _ = O.attend(rng.standard_normal((1, 4)), rng.standard_normal((1, 4)), V[:1], 0.5)
    np.testing.assert_allclose(o, V[:1], rtol=0, atol=1e-15)
    o, _ = O.attend(np.ones((3, 4)), np.zeros((0, 4)), np.zeros((0, 5)), 0.5)
    assert o.shape == (3, 5) and np.all(o == 0)


def test_round_to_bf16_matches_torch():
    rng = np.random.default_rng(14)
    x = rng.standard_normal(20000).astype(np.float32).astype(np.float64) * 10.0 ** rng.integers(-6, 6, 20000)
    x = x.astype(np.float32).astype(np.float64)   # float32-exact: one rounding in torch too
    want = torch.tensor(x, dtype=torch.float32).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(O.round_to_bf16(x), want)
    assert O.round_to_bf16(np.array([1.0 + 2.0 ** -8]))[0] == 1.0          # tie to even
    assert O.round_to_bf16(np.array([1.0 + 3 * 2.0 ** -8]))[0] == 1.0 + 2.0 ** -6


def test_log_sum_exp_closed_forms_and_normaliser():
    """The branch log-sum-exp: closed forms (n equal logits z give z + log n; one
    key gives its logit; no key gives -inf; huge logits do not overflow), and it is
    the normaliser of attend's softmax: exp(s q.k - lse) reproduces attend's
    probabilities and output."""
    rng = np.random.default_rng(11)
    q = rng.standard_normal((3, 8))
    K = np.tile(rng.standard_normal((1, 8)), (5, 1))
    z = 0.25 * (q @ K[0])
    np.testing.assert_allclose(O.log_sum_exp(q, K, 0.25), z + np.log(5.0), rtol=0, atol=1e-12)
    np.testing.assert_allclose(O.log_sum_exp(q, K[:1], 0.25), z, rtol=0, atol=1e-12)
    assert np.all(O.log_sum_exp(q, K[:0], 0.25) == -np.inf)
    big = O.log_sum_exp(np.full((1, 1), 1000.0), np.array([[1.0], [1.0]]), 1.0)
    np.testing.assert_allclose(big, 1000.0 + np.log(2.0), rtol=1e-15)
    K = rng.standard_normal((7, 8))
    V = rng.standard_normal((7, 4))
    out, p = O.attend(q, K, V, 0.3)
    lse = O.log_sum_exp(q, K, 0.3)
    p2 = np.exp(0.3 * (q @ K.T) - lse[:, None])
    np.testing.assert_allclose(p2, p, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(p2 @ V, out, rtol=1e-12, atol=1e-12)


def test_query_lse_covers_each_branch_key_set():
    """nsa_query's per-branch lse: with every block selected and a window as long as
    the prefix, the selected and window lse are the causal prefix's; the compressed
    lse is over exactly the visible blocks (-inf before the first one)."""
    rng = np.random.default_rng(12)
    T, G, dk = 40, 2, 8
    K = rng.standard_normal((T, dk))
    V = rng.standard_normal((T, 3))
    Kc = rng.standard_normal((O.n_compressed(T, 8, 4), dk))
    Vc = rng.standard_normal((Kc.shape[0], 3))
    for t in (3, 17, 39):
        qg = rng.standard_normal((G, dk))
        r = O.nsa_query(qg, K, V, Kc, Vc, t, np.ones((G, 3)), 8, 4, 8, 64, 0, 0, 64)
        s = 1 / np.sqrt(dk)
        want = O.log_sum_exp(qg, K[:t + 1], s)
        np.testing.assert_allclose(r.lse[:, 1], want, rtol=1e-12)
        np.testing.assert_allclose(r.lse[:, 2], want, rtol=1e-12)
        nvis = O.n_compressed(t + 1, 8, 4)
        if nvis == 0:
            assert np.all(r.lse[:, 0] == -np.inf)
        else:
            np.testing.assert_allclose(r.lse[:, 0], O.log_sum_exp(qg, Kc[:nvis], s), rtol=1e-12)
