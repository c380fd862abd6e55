"""GPU parity of nsa_compress_append (streaming compression in decode) against the
float64 oracle, and decode steps that rely on it."""
import numpy as np
import pytest
import torch

import long_context_sparse_nsa_amd as N
import nsa_inputs as I
from oracle import nsa_oracle as O
from tests import gpu_util as U

pytestmark = pytest.mark.gpu

STD = "decode_64k_b8"
SENTINEL = 0x3F3F  # bf16 bits of 0.746...; rows the call must not touch keep it


class Dev:
    """A case's caches and weights on the GPU, with a sentinel-filled compressed cache."""

    def __init__(self, case):
        wl, p = case.wl, case.p
        self.case = case
        self.dims, self.cfg = U.dims_cfg(case)
        self.cuc = U.cmp_offsets(case)
        self.k, self.v = U.dev_bits(case.k), U.dev_bits(case.v)
        self.wk, self.pek = U.dev_bits(case.w_k), U.dev_bits(case.pe_k)
        self.wv, self.pev = U.dev_bits(case.w_v), U.dev_bits(case.pe_v)
        self.cu = torch.from_numpy(case.cu_seqlens).cuda()
        self.cu_c = torch.from_numpy(self.cuc).cuda()
        self.max_len = int(np.diff(case.cu_seqlens).max())
        rows = max(int(wl.num_kv_heads * self.cuc[-1]), 1)
        self.kc = U.dev_bits(np.full((rows, wl.d_k), SENTINEL, np.uint16))
        self.vc = U.dev_bits(np.full((rows, wl.d_v), SENTINEL, np.uint16))
        self.ws = N.new_workspace(N.nsa_compress_append_workspace_size(self.dims, self.cfg))

    def append(self, lens):
        seq = torch.from_numpy(np.asarray(lens, dtype=np.int32)).cuda()
        N.nsa_compress_append(self.dims, self.cfg, self.k, self.v, self.cu, seq, self.max_len, self.wk, self.pek,
                              self.wv, self.pev, self.kc, self.vc, self.cu_c, self.ws)
        torch.cuda.synchronize()

    def cache_bits(self):
        return U.host_bits(self.kc), U.host_bits(self.vc)


def _due(L, p, ccap):
    if L < p.l or (L - p.l) % p.d != 0:
        return None
    i = (L - p.l) // p.d
    return i if i < ccap else None


def _assert_rows_close(got_bits, want_bits, what):
    """Same bar as the full compression: within one bf16 ulp, rarely differing."""
    got, want = U.bits_to_f64(got_bits), U.bits_to_f64(want_bits)
    ulp = np.maximum(np.abs(want), 1e-30) * 2.0 ** -7
    assert np.all(np.abs(got - want) <= ulp + 1e-6), what
    assert np.mean(got != want) < 0.05, what


def _check_append(case, dev, lens, before):
    """Due rows equal the oracle's block; every other row keeps its previous bits."""
    wl, p = case.wl, case.p
    H = wl.num_kv_heads
    kc_o, vc_o, cuc = U.oracle_cmp_cache(case)   # blocks of the full capacity: block i only reads its own tokens
    got_k, got_v = dev.cache_bits()
    exp_k, exp_v = before[0].copy(), before[1].copy()
    due_rows = []
    for b in range(wl.batch):
        ccap = int(cuc[b + 1] - cuc[b])
        i = _due(int(lens[b]), p, ccap)
        if i is None:
            continue
        for g in range(H):
            r = H * int(cuc[b]) + g * ccap + i
            due_rows.append(r)
            exp_k[r], exp_v[r] = kc_o[r], vc_o[r]
    due_rows = np.array(due_rows, dtype=np.int64)
    other = np.setdiff1d(np.arange(got_k.shape[0]), due_rows)
    assert np.array_equal(got_k[other], exp_k[other]), "rows without a due block were modified"
    assert np.array_equal(got_v[other], exp_v[other]), "rows without a due block were modified"
    if due_rows.size:
        _assert_rows_close(got_k[due_rows], exp_k[due_rows], "keys")
        _assert_rows_close(got_v[due_rows], exp_v[due_rows], "values")
    return due_rows.size


def test_append_writes_due_blocks_only():
    case = I.generate(I.workload(STD, batch=6, seq_len=3000, needles=2), 31)
    dev = Dev(case)
    p = case.p
    lens = np.array([p.l - 1, p.l, p.l + p.d, p.l + p.d + 1, 2992, 3000], dtype=np.int32)
    before = dev.cache_bits()
    dev.append(lens)
    assert _check_append(case, dev, lens, before) == 3 * case.wl.num_kv_heads


def test_append_many_rows_two_tiles():
    """80 (sequence, KV head) rows: two 64-row tiles, the second partly empty."""
    case = I.generate(I.workload(STD, batch=20, seq_len=700, ragged_min=300, needles=0), 32)
    dev = Dev(case)
    p = case.p
    rng = np.random.default_rng(5)
    caps = np.diff(case.cu_seqlens)
    lens = []
    for c in caps:
        if rng.random() < 0.7:   # a due length
            i = rng.integers(0, (int(c) - p.l) // p.d + 1)
            lens.append(int(i) * p.d + p.l)
        else:
            lens.append(int(rng.integers(1, int(c) + 1)))
    lens = np.array(lens, dtype=np.int32)
    before = dev.cache_bits()
    dev.append(lens)
    assert _check_append(case, dev, lens, before) > 0


@pytest.mark.parametrize("shape", [
    dict(d_k=64, d_v=64, num_q_heads=8, num_kv_heads=2, params=dict(l=8, d=4, l_sel=16, n_sel=8, n_local=1, w=64)),
    dict(d_k=128, d_v=128, num_q_heads=16, num_kv_heads=2, params=dict(l=16, d=8, l_sel=64, n_sel=8, w=128)),
    dict(d_k=192, d_v=128, num_q_heads=8, num_kv_heads=2, params=dict(l=6, d=2, l_sel=16, n_sel=8, w=64)),
    dict(d_k=192, d_v=128, num_q_heads=32, num_kv_heads=2, params=dict(l=64, d=32, l_sel=128, n_sel=8, w=256)),
], ids=["d64_l8", "d128_l16", "d192_l6_ragged_chunk", "d192_l64"])
def test_append_other_shapes(shape):
    """Chunk counts 2, 8, 4.5 (a partial last chunk) and 48."""
    case = I.generate(I.workload(STD, batch=3, seq_len=900, needles=0, **shape), 33)
    dev = Dev(case)
    p = case.p
    lens = np.array([p.l, 900 - (900 - p.l) % p.d, p.l + 5 * p.d], dtype=np.int32)
    before = dev.cache_bits()
    dev.append(lens)
    assert _check_append(case, dev, lens, before) == 3 * case.wl.num_kv_heads


def test_append_repeat_is_bitwise_identical():
    case = I.generate(I.workload(STD, batch=4, seq_len=2000, needles=0), 34)
    dev = Dev(case)
    lens = np.array([32, 1008, 2000, 1504], dtype=np.int32)
    dev.append(lens)
    first = dev.cache_bits()
    dev.append(lens)
    second = dev.cache_bits()
    assert np.array_equal(first[0], second[0]) and np.array_equal(first[1], second[1])


def test_serving_steps_append_then_decode():
    """Token-by-token decode: each step appends the block its token completes, then
    attends.  Outputs match the oracle (which compresses the whole prefix itself)
    at every step, and the cache grown this way matches the oracle's."""
    case = I.generate(I.workload(STD, batch=2, seq_len=2100, needles=4), 35)
    wl, p = case.wl, case.p
    dev = Dev(case)
    caps = np.diff(case.cu_seqlens).astype(np.int64)
    L0 = np.array([1990, 2001], dtype=np.int64)
    # the prompt's compressed cache, as a prefill would leave it
    seq0 = torch.from_numpy(L0.astype(np.int32)).cuda()
    N.nsa_compress_kv(dev.dims, dev.cfg, dev.k, dev.v, dev.cu, seq0, dev.max_len, dev.wk, dev.pek, dev.wv,
                      dev.pev, dev.kc, dev.vc, dev.cu_c)
    q = U.dev_bits(case.q)
    g = torch.from_numpy(np.ascontiguousarray(case.gates, dtype=np.float32)).cuda()
    out = torch.empty((wl.batch, wl.num_q_heads, wl.d_v), dtype=torch.bfloat16, device="cuda")
    sel = torch.empty((wl.batch, wl.num_kv_heads, p.n_sel), dtype=torch.int32, device="cuda")
    ws = N.new_workspace(N.nsa_decode_workspace_size(dev.dims, dev.cfg, dev.max_len))
    G = wl.num_q_heads // wl.num_kv_heads
    due_steps = 0
    for step in range(1, 41):
        lens = np.minimum(L0 + step, caps).astype(np.int32)
        dev.append(lens)
        seq = torch.from_numpy(lens).cuda()
        N.nsa_decode_fwd(dev.dims, dev.cfg, q, dev.k, dev.v, dev.kc, dev.vc, seq, dev.cu, dev.cu_c, dev.max_len,
                         g, out, sel, ws)
        torch.cuda.synchronize()
        due = [(int(L) - p.l) % p.d == 0 for L in lens]
        due_steps += any(due)
        if not (any(due) or step == 40 or step % 7 == 0):
            continue
        case.seq_lens = lens
        got = U.bits_to_f64(U.host_bits(out))
        gs = sel.cpu().numpy()
        for b in range(wl.batch):
            for gg in range(wl.num_kv_heads):
                res = O.decode_group(case, b, gg)
                t = int(lens[b]) - 1
                res = U.check_selection(res, gs[b, gg], t, p,
                                        lambda idx, b=b, gg=gg: O.decode_group(case, b, gg, override_idx=idx))
                U.assert_close(got[b, gg * G:(gg + 1) * G], res.out, f"step={step} b={b} g={gg} t={t}")
    assert due_steps >= 4
    # the grown cache: every block of the final lengths matches the oracle
    kc_o, vc_o, cuc = U.oracle_cmp_cache(case)
    got_k, got_v = dev.cache_bits()
    H = wl.num_kv_heads
    for b in range(wl.batch):
        ccap = int(cuc[b + 1] - cuc[b])
        n = O.n_compressed(int(case.seq_lens[b]), p.l, p.d)
        for gg in range(H):
            r0 = H * int(cuc[b]) + gg * ccap
            _assert_rows_close(got_k[r0:r0 + n], kc_o[r0:r0 + n], f"keys b={b} g={gg}")
            _assert_rows_close(got_v[r0:r0 + n], vc_o[r0:r0 + n], f"values b={b} g={gg}")
