"""GPU parity of nsa_decode_fwd / nsa_compress_kv against the float64 oracle."""
import numpy as np
import pytest

import long_context_sparse_nsa_amd as N
import nsa_inputs as I
from oracle import nsa_oracle as O
from tests import gpu_util as U

pytestmark = pytest.mark.gpu

STD = "decode_64k_b8"


def _check_decode(case, out, sel, groups=None, Kc_o=None, gates=None):
    """Compare every (or the given) (b, g) with the oracle."""
    wl, p = case.wl, case.p
    G = wl.num_q_heads // wl.num_kv_heads
    pairs = groups or [(b, g) for b in range(wl.batch) for g in range(wl.num_kv_heads)]
    errs = []
    for b, g in pairs:
        if gates is not None:
            saved = case.gates
            case.gates = gates
        res = O.decode_group(case, b, g)
        t = int(case.seq_lens[b]) - 1
        res = U.check_selection(res, sel[b, g], t, p, lambda idx: O.decode_group(case, b, g, override_idx=idx))
        if gates is not None:
            case.gates = saved
        errs.append(U.assert_close(out[b, g * G:(g + 1) * G], res.out, f"b={b} g={g} t={t}"))
    return errs


@pytest.mark.parametrize("seed,L", [(0, 9000), (1, 4097), (2, 20000)])
def test_decode_matches_oracle_with_oracle_cache(seed, L):
    """Decode alone: the GPU reads the oracle's compressed cache."""
    case = I.generate(I.workload(STD, batch=2, seq_len=L), seed)
    kc, vc, _ = U.oracle_cmp_cache(case)
    out, sel, _ = U.run_decode(case, kc, vc)
    _check_decode(case, out, sel)


@pytest.mark.parametrize("branch", [0, 1, 2])
def test_decode_gates_isolate_each_branch(branch):
    case = I.generate(I.workload(STD, batch=2, seq_len=6000), 10 + branch)
    gates = np.zeros_like(case.gates)
    gates[..., branch] = 1.0
    kc, vc, _ = U.oracle_cmp_cache(case)
    out, sel, _ = U.run_decode(case, kc, vc, gates=gates)
    _check_decode(case, out, sel, gates=gates)


def test_decode_end_to_end_with_gpu_compression():
    case = I.generate(I.workload(STD, batch=2, seq_len=12345), 3)
    out, sel, _ = U.run_decode(case)
    _check_decode(case, out, sel)


def test_compress_matches_oracle():
    case = I.generate(I.workload(STD, batch=2, seq_len=5000), 4)
    kc_o, vc_o, cuc = U.oracle_cmp_cache(case)
    _, _, (kc, vc) = U.run_decode(case)
    got_k = U.bits_to_f64(U.host_bits(kc))
    got_v = U.bits_to_f64(U.host_bits(vc))
    want_k, want_v = U.bits_to_f64(kc_o), U.bits_to_f64(vc_o)
    # both sides round the same real number to bf16; they may differ by one bf16 ulp
    # where the fp32 accumulation lands on the other side of a rounding midpoint
    ulp = np.maximum(np.abs(want_k), 1e-30) * 2.0 ** -7
    assert np.all(np.abs(got_k - want_k) <= ulp + 1e-6)
    assert np.mean(got_k != want_k) < 0.02
    ulpv = np.maximum(np.abs(want_v), 1e-30) * 2.0 ** -7
    assert np.all(np.abs(got_v - want_v) <= ulpv + 1e-6)


def test_decode_ragged_fine_selection():
    """Ragged lengths, l' = 32, n = 32."""
    case = I.generate(I.workload("decode_ragged_16", batch=4, seq_len=9000, ragged_min=300), 5)
    kc, vc, _ = U.oracle_cmp_cache(case)
    out, sel, _ = U.run_decode(case, kc, vc)
    _check_decode(case, out, sel)


@pytest.mark.parametrize("batch,L,rmin,seed", [(16, 20000, 1000, 51), (24, 30000, None, 52)],
                         ids=["ragged_balanced_plan", "long_batch_keeps_fixed_plan"])
def test_decode_large_batch_plans(batch, L, rmin, seed):
    """Batches whose fixed segment plan needs more than one round of workgroups.
    A ragged one is re-planned on the device from the actual lengths (segments
    of equal tile counts); one whose sequences are all long keeps the fixed plan
    (balanced segments would not fit one round either).  The GPU compresses the
    cache; the shortest and longest sequences and a few others are checked
    against the oracle in every group."""
    kw = dict(batch=batch, seq_len=L, needles=0)
    if rmin:
        kw["ragged_min"] = rmin
    case = I.generate(I.workload(STD, **kw), seed)
    out, sel, _ = U.run_decode(case)
    lens = case.seq_lens
    bs = sorted({int(np.argmin(lens)), int(np.argmax(lens)), 0, batch // 2, batch - 1})
    _check_decode(case, out, sel, groups=[(b, g) for b in bs for g in range(case.wl.num_kv_heads)])


@pytest.mark.parametrize("L", [1, 5, 31, 32, 33, 64, 65, 1024, 1025, 4096 + 16, 16 * 256 + 32])
def test_decode_edge_lengths(L):
    """No complete compressed block, exactly one, all candidates selected, chunk edges."""
    case = I.generate(I.workload(STD, batch=1, seq_len=L, needles=0), 100 + L)
    kc, vc, _ = U.oracle_cmp_cache(case)
    out, sel, _ = U.run_decode(case, kc, vc)
    _check_decode(case, out, sel)


def test_decode_small_heads_group4():
    """d_k = d_v = 64, 4 query heads per KV head (the tiny workload's head shape)."""
    wl = I.workload(STD, batch=3, seq_len=3000, num_q_heads=8, num_kv_heads=2, d_k=64, d_v=64,
                    params={"n_sel": 4, "n_local": 1, "w": 64})
    case = I.generate(wl, 6)
    kc, vc, _ = U.oracle_cmp_cache(case)
    out, sel, _ = U.run_decode(case, kc, vc)
    _check_decode(case, out, sel)


def test_decode_small_heads_many_units():
    """d_k = d_v = 64, 4 query heads per KV head, 64 ragged sequences x 2 KV heads:
    128 units, so the streaming pass takes the balanced plan and the selection
    kernel its 8-wave workgroups (one 32-token step per wave, 16 heads x 64
    channels merged by 512 threads).  Sampled sequences in every group."""
    wl = I.workload(STD, batch=64, seq_len=2600, num_q_heads=8, num_kv_heads=2, d_k=64, d_v=64,
                    ragged_min=700, needles=0, params={"n_sel": 16, "n_local": 2, "w": 512})
    case = I.generate(wl, 61)
    out, sel, _ = U.run_decode(case)
    lens = case.seq_lens
    bs = sorted({int(np.argmin(lens)), int(np.argmax(lens)), 0, 31, 63})
    _check_decode(case, out, sel, groups=[(b, g) for b in bs for g in range(2)])


def test_decode_repeat_is_bitwise_identical():
    """Same inputs twice through the same workspace: identical bits (no atomics in sums)."""
    case = I.generate(I.workload(STD, batch=2, seq_len=7000), 7)
    kc, vc, _ = U.oracle_cmp_cache(case)
    import long_context_sparse_nsa_amd as N
    dims, cfg = U.dims_cfg(case)
    ws = N.new_workspace(N.nsa_decode_workspace_size(dims, cfg, 7000))
    a = U.run_decode(case, kc, vc, ws=ws)
    b = U.run_decode(case, kc, vc, ws=ws)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


def test_decode_workspace_contents_on_entry_do_not_matter():
    """One workspace serves calls of other batch sizes and lengths in turn, and
    whatever it holds on entry (here all bytes 0xFF, or another call's data) does
    not change the result: every call is checked against the oracle."""
    a = I.generate(I.workload(STD, batch=2, seq_len=7000), 21)
    b = I.generate(I.workload(STD, batch=1, seq_len=2500), 22)
    c = I.generate(I.workload(STD, batch=3, seq_len=5000), 23)
    size = max(N.nsa_decode_workspace_size(*U.dims_cfg(x), int(np.diff(x.cu_seqlens).max())) for x in (a, b, c))
    ws = N.new_workspace(size)
    for i, case in enumerate((a, b, c, a)):
        if i % 2 == 0:
            ws.fill_(0xFF)
        kc, vc, _ = U.oracle_cmp_cache(case)
        out, sel, _ = U.run_decode(case, kc, vc, ws=ws)
        _check_decode(case, out, sel)


@pytest.mark.parametrize("params,L", [
    # selection blocks of 32 stride units (l'/d = 32 > 16 keys of a wave's row tile), keys of 2 units
    ({"l": 8, "d": 4, "l_sel": 128, "n_sel": 8, "n_local": 1, "w": 256}, 7000),
    # one stride unit per key and per block (l = d = l')
    ({"l": 16, "d": 16, "l_sel": 16, "n_sel": 16, "n_local": 2, "w": 128}, 5000),
    # compressed blocks as long as selection blocks (l = l')
    ({"l": 64, "d": 16, "l_sel": 64, "n_sel": 16, "n_local": 2, "w": 512}, 9000),
    # 8 gather workgroups and more than two window partials (the general merge)
    ({"l": 32, "d": 16, "l_sel": 64, "n_sel": 32, "n_local": 2, "w": 2048}, 9000),
])
def test_decode_block_shapes(params, L):
    """Other (l, d, l', n, w): fold geometry, partial counts and merge paths."""
    case = I.generate(I.workload(STD, batch=1, seq_len=L, params=params), 40 + L % 97)
    kc, vc, _ = U.oracle_cmp_cache(case)
    out, sel, _ = U.run_decode(case, kc, vc)
    _check_decode(case, out, sel)


@pytest.mark.parametrize("name", [STD, "decode_ragged_16"])
def test_decode_tied_scores(name):
    """Zero queries give every visible compressed block the same probability, so
    the group scores of whole selection blocks tie up to rounding: the top-n's
    tie rule and its many-survivor paths run.  The selection must be a valid
    top-n under the tie tolerance and the output must match the oracle."""
    case = I.generate(I.workload(name, batch=2, seq_len=9000, ragged_min=5000 if name != STD else None), 21)
    case.q = np.zeros_like(case.q)
    kc, vc, _ = U.oracle_cmp_cache(case)
    out, sel, _ = U.run_decode(case, kc, vc)
    _check_decode(case, out, sel)


def test_decode_two_launch_plans_each_repeat_and_match_the_oracle():
    """Two launch plans for the same inputs: the capacity the call is planned for
    (max_seq_len) sets the segment length of the compressed stream, so 4x the
    capacity splits the same cache into fewer, longer segments.  Each plan must
    repeat bit for bit, and both must match the oracle."""
    case = I.generate(I.workload(STD, batch=2, seq_len=12000), 22)
    dims, cfg = U.dims_cfg(case)
    kc, vc, _ = U.oracle_cmp_cache(case)
    cap = int(np.diff(case.cu_seqlens).max())
    sizes = []
    for max_len in (cap, 4 * cap):
        sizes.append(N.nsa_decode_workspace_size(dims, cfg, max_len))
        a = U.run_decode(case, kc, vc, max_len=max_len)
        b = U.run_decode(case, kc, vc, max_len=max_len)
        np.testing.assert_array_equal(a[0], b[0])
        np.testing.assert_array_equal(a[1], b[1])
        _check_decode(case, a[0], a[1])
    assert sizes[0] != sizes[1]  # a different segment plan
