"""The allocation-free decode entry point against nsa_decode_fwd (same kernels,
so the outputs and selections must be identical bit for bit), on two calls in a
row, the second with a smaller input, each also checked against the oracle."""
import numpy as np
import pytest
import torch

import long_context_sparse_nsa_amd as N
import nsa_inputs as I
from oracle import nsa_oracle as O
from tests import gpu_util as U

pytestmark = pytest.mark.gpu


def _upload(case):
    wl = case.wl
    dims, cfg = U.dims_cfg(case)
    cuc = U.cmp_offsets(case)
    kc_bits, vc_bits, _ = U.oracle_cmp_cache(case)
    T = dict(q=U.dev_bits(case.q), k=U.dev_bits(case.k), v=U.dev_bits(case.v), kc=U.dev_bits(kc_bits),
             vc=U.dev_bits(vc_bits), seq=torch.from_numpy(case.seq_lens).cuda(),
             cu=torch.from_numpy(case.cu_seqlens).cuda(), cuc=torch.from_numpy(cuc).cuda(),
             gates=torch.from_numpy(np.ascontiguousarray(case.gates, dtype=np.float32)).cuda())
    max_len = int(np.diff(case.cu_seqlens).max())
    return dims, cfg, T, max_len


def _outputs(case, dims, cfg):
    wl = case.wl
    out = torch.full((wl.batch, wl.num_q_heads, wl.d_v), float("nan"), dtype=torch.bfloat16, device="cuda")
    sel = torch.full((wl.batch, wl.num_kv_heads, cfg.n_sel), -7, dtype=torch.int32, device="cuda")
    return out, sel


def test_noalloc_decode_matches_the_workspace_entry_point():
    cases = [("decode_ragged_16", dict(batch=6, seq_len=20000, ragged_min=4096), 41),   # the larger call first
             ("decode_64k_b8", dict(batch=2, seq_len=7000), 42)]
    for name, kw, seed in cases:
        case = I.generate(I.workload(name, **kw), seed)
        print(f"no-alloc decode: {name} {kw} seed {seed}", flush=True)
        dims, cfg, T, max_len = _upload(case)
        ws = N.new_workspace(N.nsa_decode_workspace_size(dims, cfg, max_len))
        out_a, sel_a = _outputs(case, dims, cfg)
        out_b, sel_b = _outputs(case, dims, cfg)
        N.nsa_decode_fwd(dims, cfg, T["q"], T["k"], T["v"], T["kc"], T["vc"], T["seq"], T["cu"], T["cuc"], max_len,
                         T["gates"], out_a, sel_a, ws)
        N.nsa_decode_fwd_noalloc(dims, cfg, T["q"], T["k"], T["v"], T["kc"], T["vc"], T["seq"], T["cu"], T["cuc"],
                                 max_len, T["gates"], out_b, sel_b)
        torch.cuda.synchronize()
        assert torch.equal(out_a.view(torch.int16), out_b.view(torch.int16))
        assert torch.equal(sel_a, sel_b)
        got = U.bits_to_f64(U.host_bits(out_b))
        sel = sel_b.cpu().numpy()
        G = case.wl.num_q_heads // case.wl.num_kv_heads
        for b in range(case.wl.batch):
            for g in range(case.wl.num_kv_heads):
                res = O.decode_group(case, b, g)
                t = int(case.seq_lens[b]) - 1
                res = U.check_selection(res, sel[b, g], t, case.p,
                                        lambda idx: O.decode_group(case, b, g, override_idx=idx))
                U.assert_close(got[b, g * G:(g + 1) * G], res.out, f"no-alloc {name} b={b} g={g}")
