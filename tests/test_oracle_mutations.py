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


def test_local_blocks_skipping_one_are_caught(monkeypatch):
    """Forcing J and J - 2 instead of J and J - 1 (a plausible off-by-one in the
    trailing blocks) fails the hand example and the brute force."""
    def forced(J, n_local, fi):
        f = {0} if fi else set()
        for r in range(n_local):
            if J - 2 * r >= 0:
                f.add(J - 2 * r)
        return sorted(f)
    monkeypatch.setattr(M, "forced_blocks", forced)
    _fails(P.test_forced_blocks_hand_examples)
    with pytest.raises(AssertionError):
        for seed in range(25):
            P.test_topn_brute_force(seed)


def test_initial_block_not_forced_is_caught(monkeypatch):
    monkeypatch.setattr(M, "forced_blocks", lambda J, n_local, fi: sorted({J - r for r in range(n_local) if J - r >= 0}))
    _fails(P.test_forced_blocks_hand_examples)


# ---------------------------------------------------------------- the batch drivers

from tests import test_oracle_drivers as DR  # noqa: E402


def test_decode_driver_wrong_head_slice_is_caught(monkeypatch):
    real = M.nsa_query

    def decode_group(case, b, g, Kc=None, Vc=None, override_idx=None):
        p = case.wl.params
        G = case.wl.num_q_heads // case.wl.num_kv_heads
        K, V, Kc_o, Vc_o = M.compress_group(case, b, g)
        t = int(case.seq_lens[b]) - 1
        qg = M._widen(case.q[b, 0:G])                       # mistake: group 0's query heads
        gates = M._group_gates(case, qg, g, G, case.gates[b, g * G:(g + 1) * G])
        return real(qg, K, V, Kc_o, Vc_o, t, gates, p.l, p.d, p.l_sel, p.n_sel, p.n_local,
                    p.force_initial, p.w)
    monkeypatch.setattr(M, "decode_group", decode_group)
    _fails(DR.test_decode_driver_reads_the_documented_rows_and_heads)


def test_decode_rows_by_length_instead_of_capacity_are_caught(monkeypatch):
    def kv_rows(self, b, g):
        H = self.wl.num_kv_heads
        L = int(self.seq_lens[b])
        return H * int(self.cu_seqlens[b]) + g * L, L       # mistake: stride by the length
    monkeypatch.setattr(DR.I.Case, "kv_rows", kv_rows)
    _fails(DR.test_decode_driver_reads_the_documented_rows_and_heads)


def test_gate_network_wrong_weight_rows_are_caught(monkeypatch):
    def group_gates(case, qg, g, G, given):
        if getattr(case, "gate_net", False):
            Wg = M._widen(case.w_gate[0:G])                  # mistake: group 0's weights
            bg = np.asarray(case.b_gate[0:G], dtype=np.float64)
            return M.gate_network(qg, Wg, bg)
        return np.asarray(given, dtype=np.float64)
    monkeypatch.setattr(M, "_group_gates", group_gates)
    _fails(DR.test_decode_driver_gate_network_reads_its_heads_weights)


def test_prefill_driver_wrong_gate_slice_is_caught(monkeypatch):
    real = M.nsa_query

    def prefill_rows(case, b, g, rows, K=None, V=None, Kc=None, Vc=None, override_idx=None):
        p = case.wl.params
        G = case.wl.num_q_heads // case.wl.num_kv_heads
        K, V, Kc, Vc = M.compress_group(case, b, g)
        return [real(M._widen(case.q[b, t, g * G:(g + 1) * G]), K, V, Kc, Vc, int(t),
                     case.gates[b, t, 0:G],                  # mistake: group 0's gates
                     p.l, p.d, p.l_sel, p.n_sel, p.n_local, p.force_initial, p.w) for t in rows]
    monkeypatch.setattr(M, "prefill_rows", prefill_rows)
    _fails(DR.test_prefill_driver_reads_the_documented_rows_and_heads)


def test_dsa_driver_reading_past_the_length_is_caught(monkeypatch):
    from oracle import dsa_oracle as D

    def decode_sequence(case, b, override_idx=None):
        wl = case.wl
        t = int(case.seq_lens[b]) - 1
        cap = case.c.shape[1]
        q = D._widen_bf16(case.q[b])
        C = D._widen_bf16(case.c[b])
        kI = D.fp8_e4m3_to_float(case.k_idx[b])
        I = D.indexer_scores(D.fp8_e4m3_to_float(case.q_idx[b]), case.w_idx[b], kI)
        idx = D.topk_tokens(I, cap - 1, wl.top_k)              # mistake: the whole cache
        out, _ = M.attend(q, C[idx], C[idx][:, :wl.d_v], 1.0 / np.sqrt(C.shape[1]))
        return out, idx, I[:t + 1]
    monkeypatch.setattr(D, "decode_sequence", decode_sequence)
    _fails(DR.test_dsa_driver_reads_the_documented_rows)
