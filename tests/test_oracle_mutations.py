"""Plant plausible mistakes in the oracle (on the CPU) and check that a pin catches each.

Every mutation is applied with monkeypatch to the oracle module only and is
undone after the test; the pins themselves are the functions of
test_oracle_pins.
"""
import numpy as np
import pytest

import oracle.nsa_oracle as M
from tests import test_oracle_pins as P


def _fails(fn, *a):
    with pytest.raises(AssertionError):
        fn(*a)


def test_window_off_by_one_is_caught(monkeypatch):
    monkeypatch.setattr(M, "window_visible", lambda i, j, w: (j <= i) & (i - j <= w))
    _fails(P.test_window_mask_example)


def test_fold_normalised_by_wrong_length_is_caught(monkeypatch):
    real = M.fold_weights
    monkeypatch.setattr(M, "fold_weights", lambda n, l, d, ls, nb: real(n, l, d, ls, nb) * l / ls)
    _fails(P.test_fold_conserves_mass, 32, 16, 64)


def test_fold_dropping_the_split_half_is_caught(monkeypatch):
    real = M.fold_weights

    def drop(n, l, d, ls, nb):
        om = real(n, l, d, ls, nb)
        om[om < 1.0] = 0.0
        return om
    monkeypatch.setattr(M, "fold_weights", drop)
    _fails(P.test_fold_conserves_mass, 32, 16, 64)


def test_reversed_tie_rule_is_caught(monkeypatch):
    def sel(S, J, n, n_local, fi):
        if J + 1 <= n:
            return list(range(J + 1))
        F = M.forced_blocks(J, n_local, fi)
        rest = [j for j in range(J + 1) if j not in F]
        rest.sort(key=lambda j: (-S[j], -j))
        return sorted(F + rest[:n - len(F)])
    monkeypatch.setattr(M, "select_blocks", sel)
    _fails(P.test_topn_ties_go_to_lower_index)


def test_forced_blocks_not_counted_is_caught(monkeypatch):
    def sel(S, J, n, n_local, fi):
        if J + 1 <= n:
            return list(range(J + 1))
        F = M.forced_blocks(J, n_local, fi)
        rest = sorted((j for j in range(J + 1) if j not in F), key=lambda j: (-S[j], j))
        return sorted(F + rest[:n])
    monkeypatch.setattr(M, "select_blocks", sel)
    with pytest.raises(AssertionError):
        for seed in range(25):
            P.test_topn_brute_force(seed)


def test_channel_major_flatten_is_caught(monkeypatch):
    def compress(Kseq, W, PE, l, d, round_bf16=True):
        nc = M.n_compressed(Kseq.shape[0], l, d)
        X = np.stack([(np.asarray(Kseq[i * d:i * d + l], float) + PE).T.reshape(-1) for i in range(nc)])
        out = X @ W
        return M.round_to_bf16(out) if round_bf16 else out
    monkeypatch.setattr(M, "compress", compress)
    _fails(P.test_compression_visibility_and_flatten_order)


def test_visibility_off_by_one_is_caught(monkeypatch):
    monkeypatch.setattr(M, "n_compressed", lambda L, l, d: (L - l - 1) // d + 1 if L > l else 0)
    with pytest.raises(AssertionError):
        P.test_compression_visibility_and_flatten_order()
    _fails(P.test_nc_closed_form)


def test_missing_scale_is_caught(monkeypatch):
    real = M.attend
    monkeypatch.setattr(M, "attend", lambda q, K, V, s: real(q, K, V, 1.0))
    _fails(P.test_window_only_is_causal, 40, 8)


def test_transposed_key_operand_in_compression_is_caught(monkeypatch):
    real = M.compress
    monkeypatch.setattr(M, "compress", lambda K, W, PE, l, d, round_bf16=True:
                        real(K, W.reshape(l, K.shape[1], -1).transpose(0, 2, 1).reshape(W.shape)
                             if W.shape[1] == K.shape[1] else W, PE, l, d, round_bf16))
    _fails(P.test_compression_visibility_and_flatten_order)
