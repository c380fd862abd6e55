"""GPU parity of nsa_prefill_fwd against the float64 oracle."""
import numpy as np
import pytest

import nsa_inputs as I
from oracle import nsa_oracle as O
from tests import gpu_util as U

pytestmark = pytest.mark.gpu


def _check_rows(case, out, sel, rows, groups=None):
    wl, p = case.wl, case.p
    G = wl.num_q_heads // wl.num_kv_heads
    for b in range(wl.batch):
        for g in (groups if groups is not None else range(wl.num_kv_heads)):
            K, V, Kc, Vc = O.compress_group(case, b, g)
            res = O.prefill_rows(case, b, g, rows, K, V, Kc, Vc)
            got, want = [], []
            for t, r in zip(rows, res):
                r = U.check_selection(r, sel[b, t, g], t, p,
                                      lambda idx, t=t: O.prefill_rows(case, b, g, [t], K, V, Kc, Vc, [idx])[0])
                got.append(out[b, t, g * G:(g + 1) * G])
                want.append(r.out)
            U.assert_close(np.stack(got), np.stack(want), f"b={b} g={g}")


def test_tiny_prefill_all_rows():
    case = I.generate(I.workload("tiny_prefill_512"), 0)
    out, sel = U.run_prefill(case)
    _check_rows(case, out, sel, range(512))


@pytest.mark.parametrize("branch", [0, 1, 2])
def test_tiny_prefill_gates_isolate(branch):
    case = I.generate(I.workload("tiny_prefill_512"), 1)
    case.gates = np.zeros_like(case.gates)
    case.gates[..., branch] = 1.0
    out, sel = U.run_prefill(case)
    _check_rows(case, out, sel, range(512))


def test_prefill_wide_heads_all_rows():
    """d_k=192, d_v=128, 16 heads per group; several 64-key slices and a ragged tail."""
    case = I.generate(I.workload("prefill_32k", seq_len=1500), 2)
    out, sel = U.run_prefill(case)
    _check_rows(case, out, sel, range(1500))


def test_prefill_precomputed_cache_path():
    case = I.generate(I.workload("prefill_32k", seq_len=900), 3)
    kc, vc = [], []
    for g in range(case.wl.num_kv_heads):
        _, _, Kc, Vc = O.compress_group(case, 0, g)
        kc.append(U.f64_to_bits(Kc))
        vc.append(U.f64_to_bits(Vc))
    out, sel = U.run_prefill(case, kc_bits=np.stack(kc)[None], vc_bits=np.stack(vc)[None])
    _check_rows(case, out, sel, range(900))


def test_prefill_fine_selection_l32():
    case = I.generate(I.workload("prefill_32k", seq_len=1100, params={"l_sel": 32, "n_sel": 32}), 4)
    out, sel = U.run_prefill(case)
    _check_rows(case, out, sel, range(0, 1100, 3))


# Each branch's log-sum-exp (lse_out): the window and selected sums are those of
# the bf16 probabilities (relative error <= 2^-9 per term, so |d lse| <= 2^-9),
# the compressed one is fp32; the logits are exact products of bf16 values summed
# in fp32.  Bound: 4e-3 absolute; -inf exactly where the oracle has no key.
LSE_ABS = 4e-3


@pytest.mark.parametrize("wl_name,T,seed", [("tiny_prefill_512", 512, 5), ("prefill_32k", 1100, 6)])
def test_prefill_lse_out(wl_name, T, seed):
    case = I.generate(I.workload(wl_name, seq_len=T), seed)
    wl, p = case.wl, case.p
    G = wl.num_q_heads // wl.num_kv_heads
    _, sel, lse = U.run_prefill(case, with_lse=True)
    worst = 0.0
    for g in range(wl.num_kv_heads):
        K, V, Kc, Vc = O.compress_group(case, 0, g)
        res = O.prefill_rows(case, 0, g, range(T), K, V, Kc, Vc)
        for t, r in zip(range(T), res):
            r = U.check_selection(r, sel[0, t, g], t, p,
                                  lambda idx, t=t: O.prefill_rows(case, 0, g, [t], K, V, Kc, Vc, [idx])[0])
            got = lse[0, t, g * G:(g + 1) * G]
            want = r.lse
            assert np.array_equal(np.isneginf(got), np.isneginf(want)), (g, t)
            fin = np.isfinite(want)
            assert np.all(np.isfinite(got[fin])), (g, t)
            if fin.any():
                worst = max(worst, float(np.abs(got[fin] - want[fin]).max()))
    print(f"lse max-abs error {worst:.2e}")
    assert worst <= LSE_ABS


@pytest.mark.parametrize("wl_name,T,batch", [
    ("tiny_prefill_512", 1, 1),     # one position: window and selection hold only token 0
    ("tiny_prefill_512", 17, 1),    # shorter than one compression block: no compressed key
    ("tiny_prefill_512", 33, 1),    # the first compressed block completes at t = l - 1
    ("tiny_prefill_512", 65, 1),    # one position past a selection block and a 16-position tile
    ("tiny_prefill_512", 130, 2),   # two sequences, ragged last tile
    ("prefill_32k", 1, 1),
    ("prefill_32k", 47, 1),
    ("prefill_32k", 200, 2),
])
def test_prefill_edge_lengths(wl_name, T, batch):
    case = I.generate(I.workload(wl_name, seq_len=T, batch=batch), 11)
    print(f"[prefill edge] {wl_name} T={T} batch={batch}", flush=True)
    out, sel = U.run_prefill(case)
    _check_rows(case, out, sel, range(T))
