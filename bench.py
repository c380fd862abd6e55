#!/usr/bin/env python3
"""NSA forward-pass benchmark on one MI355X.

Headline: decode step at 64k context, batch 8, 64 query heads / 4 KV heads,
d_k=192, d_v=128, l=32, d=16, l'=64, n=16, w=512 (the compressed cache is
precomputed and resident, as in a serving loop).  One step = one
nsa_decode_fwd call = one new token for each of the 8 sequences, i.e. the whole
hot path: compressed attention, group scores, top-n, selected and window
attention, gated sum.  value = tokens/s = 8 / step time.

Timing: K back-to-back steps replayed from a HIP graph, each step on its own copy
of the KV cache (6 copies, 8.6 GB, far beyond the 256 MB Infinity Cache) so every
step reads HBM cold, bracketed by torch.cuda.synchronize().  Per-kernel durations
come from HIP start / stop events the library attaches to each decode kernel's
dispatch on the call's stream (and from events at the phase boundaries for
prefill), in an eager run queued behind a sleep kernel.

Also reported: the causal prefill of 32768 tokens (in-call compression) and the
float64 CPU oracle on a bounded sample (cpu_baseline).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16
METRIC = "NSA decode tokens/sec at 64k ctx (HBM GB/s %peak); prefill TFLOP/s (%MFMA)"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# sources of the decode kernels (a counter summary taken on other sources is not used)
DECODE_SOURCES = ("nsa_decode.hip", "nsa_tiles.hpp", "nsa_topn.hpp", "nsa_device.hpp", "nsa_internal.hpp")


def src_hash(*names) -> str:
    h = hashlib.sha256()
    for n in names:
        h.update(open(os.path.join(ROOT, "long_context_sparse_nsa_amd", "csrc", n), "rb").read())
    return h.hexdigest()[:16]


class HipEvents:
    """Raw hipEvent_t handles (the library records them; torch's Event cannot time those)."""

    def __init__(self, n):
        import ctypes
        self.ct = ctypes
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.ev = []
        for _ in range(n):
            h = ctypes.c_void_p()
            if self.hip.hipEventCreate(ctypes.byref(h)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self.ev.append(h)

    def ms(self, a, b):
        out = self.ct.c_float()
        if self.hip.hipEventElapsedTime(self.ct.byref(out), self.ev[a], self.ev[b]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(out.value)

    def close(self):
        for h in self.ev:
            self.hip.hipEventDestroy(h)


def upload_case(case, torch, N):
    """Device tensors of a decode case plus its GPU-computed compressed cache."""
    wl, p = case.wl, case.p

    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()

    dims = N.make_dims(wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.d_k, wl.d_v)
    cfg = N.make_config(p.l, p.d, p.l_sel, p.n_sel, p.n_local, p.force_initial, p.w)
    caps = np.diff(case.cu_seqlens)
    ncap = np.array([N.compressed_count(int(c), p.l, p.d) for c in caps], dtype=np.int64)
    cuc = np.zeros(len(caps) + 1, dtype=np.int64)
    cuc[1:] = np.cumsum(ncap)
    T = dict(q=dev(case.q), k=dev(case.k), v=dev(case.v), w_k=dev(case.w_k), pe_k=dev(case.pe_k),
             w_v=dev(case.w_v), pe_v=dev(case.pe_v),
             gates=torch.from_numpy(case.gates).cuda(), seq=torch.from_numpy(case.seq_lens).cuda(),
             cu=torch.from_numpy(case.cu_seqlens).cuda(), cuc=torch.from_numpy(cuc).cuda())
    rows = int(wl.num_kv_heads * cuc[-1])
    T["kc"] = torch.zeros((max(rows, 1), wl.d_k), dtype=torch.bfloat16, device="cuda")
    T["vc"] = torch.zeros((max(rows, 1), wl.d_v), dtype=torch.bfloat16, device="cuda")
    max_len = int(caps.max())
    N.nsa_compress_kv(dims, cfg, T["k"], T["v"], T["cu"], T["seq"], max_len, T["w_k"], T["pe_k"], T["w_v"],
                      T["pe_v"], T["kc"], T["vc"], T["cuc"])
    torch.cuda.synchronize()
    return dims, cfg, T, max_len, cuc


def decode_bytes(case, sel):
    """Algorithmic HBM bytes of one decode step, of its first kernel and of the
    selected and window tokens.

    Step: the compressed cache, the union of selected and window tokens (each
    read once), q, gates, out.  First kernel (compressed-branch and window
    workgroups of the streaming pass): the compressed cache, the window tokens,
    q."""
    wl, p = case.wl, case.p
    row = 2 * (wl.d_k + wl.d_v)
    cmp_b, sw_b, w_b = 0, 0, 0
    for b in range(wl.batch):
        L = int(case.seq_lens[b])
        t = L - 1
        nc = (L - p.l) // p.d + 1 if L >= p.l else 0
        for g in range(wl.num_kv_heads):
            cmp_b += nc * row
            win = set(range(max(0, t - p.w + 1), t + 1))
            toks = set(win)
            for j in sel[b, g]:
                if j >= 0:
                    toks.update(range(j * p.l_sel, min((j + 1) * p.l_sel, L)))
            sw_b += len(toks) * row
            w_b += len(win) * row
    io = wl.batch * wl.num_q_heads * (wl.d_k * 2 + 3 * 4 + wl.d_v * 2)
    q_bytes = wl.batch * wl.num_q_heads * wl.d_k * 2
    return cmp_b + sw_b + io, cmp_b + w_b + q_bytes, sw_b


def graph_of_steps(torch, step, idx):
    """A HIP graph of the decode steps step(i) for i in idx (captured once, replayed)."""
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for i in idx:
                step(i)
    torch.cuda.synchronize()
    return g


def time_graph(torch, g, reps=3):
    """Median over reps of one replay's elapsed time (ms), each replay bracketed by
    events with a synchronisation on both sides; also the wall time of the first."""
    times, wall = [], None
    for r in range(reps):
        torch.cuda.synchronize()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        w0 = time.perf_counter()
        ev0.record()
        g.replay()
        ev1.record()
        torch.cuda.synchronize()
        if wall is None:
            wall = time.perf_counter() - w0
        times.append(ev0.elapsed_time(ev1))
    return float(np.median(times)), wall


def bench_decode(args, torch, N, I, name, case=None, headline=False):
    """One decode workload: K steps replayed from a graph over rotating cache copies
    (cold caches: the copies exceed the 256 MB Infinity Cache), the same K steps on
    one copy (warm), 100 steps timed one by one (median, p10, p90), and the two
    kernels' own durations from events attached to their dispatches."""
    wl = I.workload(name)
    seed = list(I.WORKLOADS).index(name)
    if case is None:
        t0 = time.time()
        case = I.generate(wl, seed)
        log(f"[bench] generated {wl.name} (seed {seed}) in {time.time() - t0:.1f}s")
    dims, cfg, T, max_len, cuc = upload_case(case, torch, N)
    ws = N.new_workspace(N.nsa_decode_workspace_size(dims, cfg, max_len))
    out = torch.empty((wl.batch, wl.num_q_heads, wl.d_v), dtype=torch.bfloat16, device="cuda")
    sel = torch.full((wl.batch, wl.num_kv_heads, cfg.n_sel), -1, dtype=torch.int32, device="cuda")
    copies = [(T["k"], T["v"], T["kc"], T["vc"])]
    for _ in range(args.copies - 1):
        copies.append(tuple(x.clone() for x in copies[0]))
    torch.cuda.synchronize()
    log(f"[bench] {wl.name}: {len(copies)} cache copies resident "
        f"({sum(x.numel() * 2 for x in copies[0]) * len(copies) / 1e9:.1f} GB)")

    def step(i):
        k, v, kc, vc = copies[i % len(copies)]
        N.nsa_decode_fwd(dims, cfg, T["q"], k, v, kc, vc, T["seq"], T["cu"], T["cuc"], max_len, T["gates"], out,
                         sel, ws)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ref_out = out.clone()
    K = args.steps
    g = graph_of_steps(torch, step, range(K))
    g.replay()
    torch.cuda.synchronize()
    if not torch.equal(out, ref_out):
        raise RuntimeError("graph replay differs from eager result")
    total_ms, wall = time_graph(torch, g)
    if not torch.equal(out, ref_out):
        raise RuntimeError("graph replay differs from eager result")
    ms_step = total_ms / K
    gw = graph_of_steps(torch, step, [0] * K)  # warm: every step on the same copy
    warm_ms = time_graph(torch, gw)[0] / K
    del g, gw

    # 100 steps timed one by one (eager, queued behind a sleep so that the GPU
    # runs them back to back), each on the next cache copy
    n_one = 100
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_one)]
    torch.cuda.synchronize()
    torch.cuda._sleep(int(2e7))
    for i in range(n_one):
        evs[i][0].record()
        step(i)
        evs[i][1].record()
    torch.cuda.synchronize()
    one = np.array([a.elapsed_time(b) for a, b in evs]) * 1e3
    dist = {"median_us": float(np.median(one)), "p10_us": float(np.percentile(one, 10)),
            "p90_us": float(np.percentile(one, 90)), "samples": n_one}

    # the kernels' own durations: events attached to each dispatch (eager, queued behind a sleep)
    n_ph = 60
    hev = HipEvents(4 * n_ph)
    torch.cuda.synchronize()
    torch.cuda._sleep(int(2e7))
    try:
        for i in range(n_ph):
            N.nsa_set_phase_events(hev.ev[4 * i:4 * i + 4])
            step(i)
    finally:
        N.nsa_set_phase_events(None)
    torch.cuda.synchronize()
    ph = [float(np.mean([hev.ms(4 * i + k, 4 * i + k + 1) for i in range(n_ph)])) for k in (0, 2)]
    hev.close()
    p1, p2 = ph
    sel_h = sel.cpu().numpy()
    b_step, b_cmp, b_sw = decode_bytes(case, sel_h)
    gbs_step = b_step / (ms_step * 1e-3) / 1e9
    gbs_cmp = b_cmp / (p1 * 1e-3) / 1e9
    res = dict(
        workload=wl.name, ms_per_step=ms_step, wall_s=wall, steps=K, timing="hip_graph",
        tokens_per_s=wl.batch / (ms_step * 1e-3), warm_ms_per_step=warm_ms, step_distribution=dist,
        step_bytes=b_step, step_gbs=gbs_step, step_frac=gbs_step / HBM_PEAK_GBS,
        pass1_us=p1 * 1e3, pass2_us=p2 * 1e3, pass1_bytes=b_cmp, pass2_bytes=b_sw,
        finish_us=p2 * 1e3, pass1_gbs=gbs_cmp, pass2_gbs=b_sw / (p2 * 1e-3) / 1e9,
        needle_hit_gpu=needle_hits(case, sel_h))
    log(f"[bench] decode {wl.name}: {ms_step * 1e3:.1f} us/step over {K} steps (warm {warm_ms * 1e3:.1f}; one by one "
        f"median {dist['median_us']:.1f}, p10 {dist['p10_us']:.1f}, p90 {dist['p90_us']:.1f}), "
        f"{res['tokens_per_s']:.4g} tok/s, {gbs_step:.0f} GB/s step ({100 * gbs_step / HBM_PEAK_GBS:.1f}%); "
        f"kernels: stream {p1 * 1e3:.1f} us ({gbs_cmp:.0f} GB/s), selection {p2 * 1e3:.1f} us")
    if not headline:
        return case, res, T
    res["phase_clock_us"] = decode_phase_clock(torch, N, step)
    log("[bench] decode phase clock (us after the first streaming workgroup starts; median / max over "
        "workgroups): " + ", ".join(f"{k} {v['median_us']}/{v['max_us']}" for k, v in res["phase_clock_us"].items()))
    res["gate_network_ms_per_step"] = bench_gate_network(args, torch, N, case, dims, cfg, T, max_len, copies,
                                                         out, sel, ws)
    log(f"[bench] decode step with the gate network: {res['gate_network_ms_per_step'] * 1e3:.1f} us")
    if not args.no_serving:
        res["serving"] = bench_serving(args, torch, N, case, dims, cfg, T, max_len, copies, step)
    return case, res, T


def needle_hits(case, sel):
    """Fraction of the planted needle blocks (l'-aligned) that a selection [B, H, n] took."""
    p = case.p
    H = case.wl.num_kv_heads
    hit = tot = 0
    for b in range(case.wl.batch):
        for g in range(H):
            picks = set(int(j) for j in sel[b, g] if j >= 0)
            nb = case.needle_blocks[b * H + g]
            tot += len(nb)
            hit += sum(1 for j in nb if int(j) in picks)
    return hit / tot if tot else None


CLK_SLOTS, CLK_GROUPS = 16, 4096
K1_PHASES = {0: "start", 1: "last_tile", 3: "waves_done", 4: "outputs_merged", 2: "stored"}
K2_PHASES = {0: "start", 1: "loads_arrived", 2: "scores_ready", 3: "topn_done", 4: "steps_done",
             5: "partials_stored", 6: "merge_start", 7: "out_written"}


DSA_K0_PHASES = {0: "start", 1: "bound", 2: "arrived", 3: "candidates_loaded", 4: "bitmaps", 5: "written",
                 6: "written_full_select"}
DSA_K1_PHASES = {0: "start", 1: "rows_loaded", 2: "first_tile", 3: "tiles_done", 4: "stored"}


def decode_phase_clock(torch, N, step, n_steps=12, kernels=((0, "stream", K1_PHASES), (1, "select", K2_PHASES))):
    """Per-workgroup phase clock of two kernels of a step (the library's profiling
    hook: thread 0 of every workgroup stamps the 100 MHz constant clock at numbered
    points), over eager steps.  Returns, per phase, the median over steps of the
    median and the maximum over workgroups of (stamp - first start of the step's
    first recorded kernel), in microseconds."""
    buf = torch.zeros(2 * CLK_GROUPS * CLK_SLOTS, dtype=torch.int64, device="cuda")
    N.nsa_set_phase_clock(buf)
    per = {}
    try:
        for i in range(n_steps):
            buf.zero_()
            torch.cuda.synchronize()
            step(i)
            torch.cuda.synchronize()
            a = buf.view(2, CLK_GROUPS, CLK_SLOTS).cpu().numpy()
            starts = a[0, :, 0]
            t0 = starts[starts > 0].min()
            for k, kname, names in kernels:
                for s, nm in names.items():
                    v = a[k, :, s]
                    v = v[v > 0]
                    if v.size:
                        d = (v - t0) / 100.0  # 100 MHz ticks -> us
                        per.setdefault(f"{kname}.{nm}", []).append((float(np.median(d)), float(d.max())))
    finally:
        N.nsa_set_phase_clock(None)
    out = {}
    for key, vals in per.items():
        vals = np.array(vals)
        out[key] = {"median_us": round(float(np.median(vals[:, 0])), 2), "max_us": round(float(np.median(vals[:, 1])), 2)}
    return out


def bench_gate_network(args, torch, N, case, dims, cfg, T, max_len, copies, out, sel, ws):
    """Decode step with the gates computed in the selection kernel from each query head
    (gate network weights instead of gate values), graph-replayed like the headline."""
    wg = torch.from_numpy(np.ascontiguousarray(case.w_gate).view(np.int16)).view(torch.bfloat16).cuda()
    bgt = torch.from_numpy(case.b_gate).cuda()

    def step(i):
        k, v, kc, vc = copies[i % len(copies)]
        N.nsa_decode_fwd(dims, cfg, T["q"], k, v, kc, vc, T["seq"], T["cu"], T["cuc"], max_len, None, out, sel, ws,
                         w_gate=wg, b_gate=bgt)

    for i in range(len(copies)):
        step(i)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for i in range(len(copies)):
                step(i)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    reps = max(1, (args.steps + len(copies) - 1) // len(copies))
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(reps):
        g.replay()
    ev1.record()
    torch.cuda.synchronize()
    return ev0.elapsed_time(ev1) / (reps * len(copies))


def append_bytes(case):
    """Algorithmic HBM bytes of one nsa_compress_append call: both weight matrices and
    position embeddings, the l tokens of every due block, the new compressed rows."""
    wl, p = case.wl, case.p
    w = 2 * p.l * (wl.d_k * wl.d_k + wl.d_v * wl.d_v) + 2 * p.l * (wl.d_k + wl.d_v)
    due = sum(1 for L in case.seq_lens if int(L) >= p.l and (int(L) - p.l) % p.d == 0)
    rows = due * wl.num_kv_heads
    return w + rows * (p.l + 1) * 2 * (wl.d_k + wl.d_v), rows


def bench_serving(args, torch, N, case, dims, cfg, T, max_len, copies, step):
    """Serving step = nsa_compress_append (the block the new token completes) +
    nsa_decode_fwd, replayed from a graph over the cache copies.  At the headline
    lengths every sequence completes a block at this step (it happens every d steps),
    so this is the step with the most append work."""
    ws_a = N.new_workspace(N.nsa_compress_append_workspace_size(dims, cfg))

    def append(i):
        k, v, kc, vc = copies[i % len(copies)]
        N.nsa_compress_append(dims, cfg, k, v, T["cu"], T["seq"], max_len, T["w_k"], T["pe_k"], T["w_v"], T["pe_v"],
                              kc, vc, T["cuc"], ws_a)

    for i in range(len(copies)):
        append(i)
        step(i)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for i in range(len(copies)):
                append(i)
                step(i)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    reps = max(1, (args.steps + len(copies) - 1) // len(copies))
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(reps):
        g.replay()
    ev1.record()
    torch.cuda.synchronize()
    ms_step = ev0.elapsed_time(ev1) / (reps * len(copies))
    # the append alone, eager, each call bracketed by events on its stream (queued behind a sleep)
    n = 30
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    torch.cuda._sleep(int(2e7))
    for i in range(n):
        evs[i][0].record()
        append(i)
        evs[i][1].record()
        step(i)  # the decode between appends evicts W from the caches, as in serving
    torch.cuda.synchronize()
    a_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    nbytes, rows = append_bytes(case)
    res = dict(ms_per_step=ms_step, tokens_per_s=case.wl.batch / (ms_step * 1e-3), append_us=a_ms * 1e3,
               append_bytes=nbytes, append_rows=rows, append_gbs=nbytes / (a_ms * 1e-3) / 1e9)
    res["append_hbm_frac"] = res["append_gbs"] / HBM_PEAK_GBS
    log(f"[bench] serving step (append + decode): {ms_step * 1e3:.1f} us; append {a_ms * 1e3:.1f} us "
        f"({rows} blocks, {res['append_gbs']:.0f} GB/s)")
    return res


def prefill_flops(wl):
    """Algorithmic FLOPs of the causal prefill (2*(d_k+d_v) per key visit per head)."""
    p = wl.params
    T = wl.seq_len
    t = np.arange(T, dtype=np.int64)
    nc = np.where(t + 1 >= p.l, (t + 1 - p.l) // p.d + 1, 0)
    J = t // p.l_sel
    sel = np.where(J + 1 <= p.n_sel, t + 1, (p.n_sel - 1) * p.l_sel + (t % p.l_sel) + 1)
    win = np.minimum(p.w, t + 1)
    per = 2 * (wl.d_k + wl.d_v) * wl.num_q_heads * wl.batch
    ncmp = (T - p.l) // p.d + 1 if T >= p.l else 0
    comp = 2 * wl.batch * wl.num_kv_heads * ncmp * p.l * (wl.d_k * wl.d_k + wl.d_v * wl.d_v)
    return dict(cmp=float(per * nc.sum()), slc=float(per * sel.sum()), win=float(per * win.sum()),
                compress=float(comp))


def backward_flops(wl):
    """Algorithmic FLOPs of the prefill backward: per key visit per head, the five
    products of an attention backward (logits again, dO.v, dq, dk: 2*d_k each;
    dO.v and dv: 2*d_v each) = 2*(3*d_k + 2*d_v); the compression backward is
    twice the compression's products (dX = dY W^T and dW)."""
    f = prefill_flops(wl)
    visits = (f["cmp"] + f["slc"] + f["win"]) / (2 * (wl.d_k + wl.d_v))
    return dict(attention=float(visits * 2 * (3 * wl.d_k + 2 * wl.d_v)), compress=float(2 * f["compress"]))


def backward_setup(torch, N, I):
    """prefill_32k inputs resident on the GPU, the compressed cache, the forward's
    selection and per-branch log-sum-exp, an output gradient and the backward's buffers."""
    wl = I.workload("prefill_32k")
    seed = list(I.WORKLOADS).index("prefill_32k")
    case = I.generate(wl, seed)
    p = wl.params
    B, T, Hq, H, dk, dv = wl.batch, wl.seq_len, wl.num_q_heads, wl.num_kv_heads, wl.d_k, wl.d_v
    nc = N.compressed_count(T, p.l, p.d)

    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()

    dims = N.make_dims(B, Hq, H, dk, dv)
    cfg = N.make_config(p.l, p.d, p.l_sel, p.n_sel, p.n_local, p.force_initial, p.w)
    dout_bits = I.output_gradient(case, seed)
    X = dict(q=dev(case.q), k=dev(case.k), v=dev(case.v), wk=dev(case.w_k), pk=dev(case.pe_k), wv=dev(case.w_v),
             pv=dev(case.pe_v), gates=torch.from_numpy(case.gates).cuda(), dout=dev(dout_bits))
    X["kc"] = torch.empty((B, H, nc, dk), dtype=torch.bfloat16, device="cuda")
    X["vc"] = torch.empty((B, H, nc, dv), dtype=torch.bfloat16, device="cuda")
    N.nsa_compress_kv(dims, cfg, X["k"], X["v"], None, None, T, X["wk"], X["pk"], X["wv"], X["pv"], X["kc"], X["vc"],
                      None)
    X["sel"] = torch.empty((B, T, H, p.n_sel), dtype=torch.int32, device="cuda")
    out = torch.empty((B, T, Hq, dv), dtype=torch.bfloat16, device="cuda")
    ws = N.new_workspace(N.nsa_prefill_workspace_size(dims, cfg, T, False))
    X["lse"] = torch.empty((B, T, Hq, 3), dtype=torch.float32, device="cuda")
    N.nsa_prefill_fwd(dims, cfg, T, X["q"], X["k"], X["v"], X["kc"], X["vc"], None, None, None, None, X["gates"],
                      out, X["sel"], ws, lse_out=X["lse"])
    f32 = lambda *sh: torch.empty(sh, dtype=torch.float32, device="cuda")
    X.update(dq=f32(B, T, Hq, dk), dk=f32(B, H, T, dk), dv=f32(B, H, T, dv), dkc=f32(B, H, nc, dk),
             dvc=f32(B, H, nc, dv), dg=f32(B, T, Hq, 3), dwk=f32(p.l * dk, dk), dpk=f32(p.l, dk),
             dwv=f32(p.l * dv, dv), dpv=f32(p.l, dv))
    X["ws"] = N.new_workspace(N.nsa_prefill_bwd_workspace_size(dims, cfg, T))
    X["wsc"] = N.new_workspace(max(N.nsa_compress_bwd_workspace_size(dims, cfg, T, w) for w in (0, 1)))
    torch.cuda.synchronize()

    def attn(saved_lse=True):  # with the forward's log-sum-exp: one pass on the query side
        N.nsa_prefill_bwd(dims, cfg, T, X["q"], X["k"], X["v"], X["kc"], X["vc"], X["gates"], X["sel"], X["dout"],
                          X["dq"], X["dk"], X["dv"], X["dkc"], X["dvc"], X["dg"], X["ws"],
                          lse=X["lse"] if saved_lse else None)

    def comp():
        N.nsa_compress_bwd(dims, cfg, T, 0, X["k"], X["wk"], X["pk"], X["dkc"], X["dk"], X["dwk"], X["dpk"], X["wsc"])
        N.nsa_compress_bwd(dims, cfg, T, 1, X["v"], X["wv"], X["pv"], X["dvc"], X["dv"], X["dwv"], X["dpv"], X["wsc"])

    return wl, attn, comp, case, dout_bits


def backward_cpu_baseline(case, dout_bits, torch):
    """The float64 backward oracle (autograd through every branch and the
    compression) on a bounded sample: the last position of KV group 0, its
    selection taken by the oracle itself."""
    from oracle import nsa_backward as NB
    wl = case.wl
    G = wl.num_q_heads // wl.num_kv_heads
    w = lambda bits: (np.asarray(bits).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    t = wl.seq_len - 1
    t0 = time.perf_counter()
    NB.sequence_backward(w(case.q[0, :, :G]), w(case.k[0, 0]), w(case.v[0, 0]), w(case.w_k), w(case.pe_k),
                         w(case.w_v), w(case.pe_v), np.asarray(case.gates[0, :, :G], dtype=np.float64),
                         w(dout_bits[0, :, :G]), [t], case.p)
    el = time.perf_counter() - t0
    # one position of one group: a position of all wl.num_kv_heads groups costs that many times more
    return dict(value=1.0 / (el * wl.num_kv_heads), unit="positions/s", cores=int(torch.get_num_threads()),
                kind="oracle", sample=f"position {t} of {wl.name}, KV group 0 of {wl.num_kv_heads} (dq, dk, dv, "
                                      f"compression and gate gradients, oracle selection); {el:.1f} s of CPU work")


def bench_backward(args, torch, N, I):
    t0 = time.time()
    wl, attn, comp, case, dout_bits = backward_setup(torch, N, I)
    log(f"[bench] backward inputs of {wl.name} ready in {time.time() - t0:.1f}s")
    attn()
    comp()
    torch.cuda.synchronize()
    reps = args.prefill_reps
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    ev[0].record()
    for _ in range(reps):
        attn()
    ev[1].record()
    for _ in range(reps):
        comp()
    ev[2].record()
    torch.cuda.synchronize()
    attn_ms, comp_ms = ev[0].elapsed_time(ev[1]) / reps, ev[1].elapsed_time(ev[2]) / reps
    attn(False)  # the same call without the saved log-sum-exp (query side in two passes)
    ev[0].record()
    for _ in range(reps):
        attn(False)
    ev[1].record()
    torch.cuda.synchronize()
    recompute_ms = ev[0].elapsed_time(ev[1]) / reps
    hev = HipEvents(4 * reps)
    try:
        for i in range(reps):
            N.nsa_set_phase_events(hev.ev[4 * i:4 * i + 4])
            attn()
        N.nsa_set_phase_events(None)
        torch.cuda.synchronize()
        ph = [float(np.median([hev.ms(4 * i + a, 4 * i + a + 1) for i in range(reps)])) for a in range(3)]
    finally:
        N.nsa_set_phase_events(None)
        hev.close()
    f = backward_flops(wl)
    ms = attn_ms + comp_ms
    res = dict(workload=wl.name, ms=ms, attention_ms=attn_ms, compress_ms=comp_ms, recompute_ms=recompute_ms, flops=f,
               tflops=(f["attention"] + f["compress"]) / (ms * 1e-3) / 1e12,
               attention_tflops=f["attention"] / (attn_ms * 1e-3) / 1e12,
               kernel_ms=dict(bwd_query_kernel=ph[0], bwd_kv_kernel_raw=ph[1], bwd_kv_kernel_cmp=ph[2]))
    res["mfma_frac"] = res["attention_tflops"] / MFMA_BF16_PEAK_TFLOPS
    log(f"[bench] backward {wl.name}: {ms:.2f} ms ({res['tflops']:.1f} TFLOP/s); attention {attn_ms:.2f} ms "
        f"({res['attention_tflops']:.0f} TFLOP/s, {100 * res['mfma_frac']:.1f}% of bf16 peak): query side "
        f"{ph[0]:.2f} ms, raw keys {ph[1]:.2f} ms, compressed keys {ph[2]:.2f} ms; compression {comp_ms:.2f} ms; "
        f"without the saved lse {recompute_ms:.2f} ms")
    res["positions_per_s"] = wl.batch * wl.seq_len / (ms * 1e-3)
    if not args.no_cpu:
        res["cpu"] = backward_cpu_baseline(case, dout_bits, torch)
        log(f"[bench] backward cpu oracle: {res['cpu']['value']:.3g} positions/s on {res['cpu']['cores']} threads")
    return res


def bench_prefill(args, torch, N, I):
    wl = I.workload("prefill_32k")
    seed = list(I.WORKLOADS).index("prefill_32k")
    t0 = time.time()
    case = I.generate(wl, seed)
    log(f"[bench] generated {wl.name} in {time.time() - t0:.1f}s")
    p = wl.params

    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()

    dims = N.make_dims(wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.d_k, wl.d_v)
    cfg = N.make_config(p.l, p.d, p.l_sel, p.n_sel, p.n_local, p.force_initial, p.w)
    q, k, v = dev(case.q), dev(case.k), dev(case.v)
    wk, pk, wv, pv = dev(case.w_k), dev(case.pe_k), dev(case.w_v), dev(case.pe_v)
    gates = torch.from_numpy(case.gates).cuda()
    out = torch.empty((wl.batch, wl.seq_len, wl.num_q_heads, wl.d_v), dtype=torch.bfloat16, device="cuda")
    ws = N.new_workspace(N.nsa_prefill_workspace_size(dims, cfg, wl.seq_len, True))

    def run():
        N.nsa_prefill_fwd(dims, cfg, wl.seq_len, q, k, v, None, None, wk, pk, wv, pv, gates, out, None, ws)

    run()
    torch.cuda.synchronize()
    reps = args.prefill_reps
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(reps):
        run()
    ev1.record()
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / reps
    # per-kernel durations from the library's phase events (compression, compressed +
    # window + top-n kernel, selected-branch kernel)
    hev = HipEvents(4 * reps)
    try:
        for i in range(reps):
            N.nsa_set_phase_events(hev.ev[4 * i:4 * i + 4])
            run()
        N.nsa_set_phase_events(None)
        torch.cuda.synchronize()
        ph = [float(np.median([hev.ms(4 * i + a, 4 * i + a + 1) for i in range(reps)])) for a in range(3)]
    finally:
        N.nsa_set_phase_events(None)
        hev.close()
    f = prefill_flops(wl)
    tot = sum(f.values())
    res = dict(workload=wl.name, ms=ms, flops=f, tflops=tot / (ms * 1e-3) / 1e12,
               mfma_frac=tot / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
               kernel_ms=dict(compress=ph[0], pf_cmp_win_kernel=ph[1], pf_sel_kernel=ph[2]),
               cmp_win_tflops=(f["cmp"] + f["win"]) / (ph[1] * 1e-3) / 1e12,
               sel_tflops=f["slc"] / (ph[2] * 1e-3) / 1e12)
    res["sel_mfma_frac"] = res["sel_tflops"] / MFMA_BF16_PEAK_TFLOPS
    # reuse of the staged selected blocks: the selection of one more call, per tile of
    # positions: the union of the tile's selected blocks (one staged copy each) against
    # the positions that use them
    sel = torch.empty((wl.batch, wl.seq_len, wl.num_kv_heads, p.n_sel), dtype=torch.int32, device="cuda")
    N.nsa_prefill_fwd(dims, cfg, wl.seq_len, q, k, v, None, None, wk, pk, wv, pv, gates, out, sel, ws)
    torch.cuda.synchronize()
    res["selected_reuse"] = selection_reuse(sel.cpu().numpy(), p)
    log("[bench] prefill selected-block reuse: " + ", ".join(
        f"{k}: union {v['mean_union_blocks']:.1f} blocks, {v['positions_per_staged_block']:.2f} positions per block"
        for k, v in res["selected_reuse"].items()))
    # the same call with the gates computed in the kernels by the gate network
    wg = dev(case.w_gate)
    bgt = torch.from_numpy(case.b_gate).cuda()

    def run_gn():
        N.nsa_prefill_fwd(dims, cfg, wl.seq_len, q, k, v, None, None, wk, pk, wv, pv, None, out, None, ws,
                          w_gate=wg, b_gate=bgt)

    run_gn()
    torch.cuda.synchronize()
    ev0.record()
    for _ in range(reps):
        run_gn()
    ev1.record()
    torch.cuda.synchronize()
    res["gate_network_ms"] = ev0.elapsed_time(ev1) / reps
    log(f"[bench] prefill with the gate network: {res['gate_network_ms']:.2f} ms")
    log(f"[bench] prefill {wl.name}: {ms:.2f} ms, {res['tflops']:.1f} TFLOP/s ({100 * res['mfma_frac']:.1f}% of bf16 "
        f"peak); compress {ph[0]:.3f} ms, cmp+win+top-n {ph[1]:.3f} ms ({res['cmp_win_tflops']:.0f} TFLOP/s), "
        f"selected {ph[2]:.3f} ms ({res['sel_tflops']:.0f} TFLOP/s, {100 * res['sel_mfma_frac']:.1f}%)")
    return res


def selection_reuse(sel, p, tiles=(8, 16, 32, 64)):
    """For position tiles of each size: the mean number of distinct selected blocks of a
    tile (the blocks one workgroup stages per (sequence, KV group)) and the positions
    served per staged block (selections made in the tile / distinct blocks), over every
    tile of every sequence and KV group.  sel is [B, T, H, n], -1 padded."""
    B, T, H, n = sel.shape
    out = {}
    for tile in tiles:
        nt = T // tile
        uni = used = 0
        for b in range(B):
            for g in range(H):
                s = sel[b, :nt * tile, g].reshape(nt, tile * n)
                for row in s:
                    v = row[row >= 0]
                    uni += np.unique(v).size
                    used += v.size
        out[f"tile_{tile}"] = {"mean_union_blocks": uni / (B * H * nt), "positions_per_staged_block": used / uni}
    return out


def dsa_upload(case, torch, N):
    wl = case.wl

    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()

    dims = N.make_dsa_dims(wl.batch, wl.num_heads, wl.d_qk, wl.d_v, wl.idx_heads, wl.idx_dim)
    T = dict(q=dev(case.q), c=dev(case.c), qi=torch.from_numpy(case.q_idx).cuda(),
             ki=torch.from_numpy(case.k_idx).cuda(), wi=torch.from_numpy(case.w_idx).cuda(),
             seq=torch.from_numpy(case.seq_lens).cuda())
    return dims, T


def dsa_bytes(case):
    """Algorithmic HBM bytes of one DSA decode step: every indexer key of the
    context, the selected tokens' latents, q (both), the indexer weights, out."""
    wl = case.wl
    keys = sum(int(L) for L in case.seq_lens) * wl.idx_dim
    sel = sum(min(int(L), wl.top_k) for L in case.seq_lens) * wl.d_qk * 2
    io = wl.batch * (wl.num_heads * (wl.d_qk + wl.d_v) * 2 + wl.idx_heads * (wl.idx_dim + 4))
    return keys, sel, keys + sel + io


def bench_dsa(args, torch, N, I):
    """DSA decode step (second workload): graph replays over rotating cache copies."""
    wl = I.dsa_workload("dsa_decode_64k_b8")
    t0 = time.time()
    case = I.generate_dsa(wl, list(I.DSA_WORKLOADS).index(wl.name))
    log(f"[bench] generated {wl.name} in {time.time() - t0:.1f}s")
    dims, T = dsa_upload(case, torch, N)
    cap, k = wl.seq_len, wl.top_k
    ws = N.new_workspace(N.nsa_dsa_decode_workspace_size(dims, k, cap))
    out = torch.empty((wl.batch, wl.num_heads, wl.d_v), dtype=torch.bfloat16, device="cuda")
    copies = [(T["c"], T["ki"])] + [(T["c"].clone(), T["ki"].clone()) for _ in range(args.copies - 1)]

    def step(i):
        c, ki = copies[i % len(copies)]
        N.nsa_dsa_decode_fwd(dims, k, T["q"], T["qi"], T["wi"], c, ki, T["seq"], cap, out, None, ws)

    for i in range(len(copies)):
        step(i)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        with torch.cuda.graph(g, stream=st):
            for i in range(len(copies)):
                step(i)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    reps = max(1, (args.steps + len(copies) - 1) // len(copies))
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(reps):
        g.replay()
    ev1.record()
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / (reps * len(copies))
    # per-phase durations: events before the indexer, after it, after the selection, at the end
    n_ph = 30
    hev = HipEvents(4 * n_ph)
    try:
        torch.cuda._sleep(int(2e7))
        for i in range(n_ph):
            N.nsa_set_phase_events(hev.ev[4 * i:4 * i + 4])
            step(i)
        N.nsa_set_phase_events(None)
        torch.cuda.synchronize()
        ph = [float(np.mean([hev.ms(4 * i + a, 4 * i + a + 1) for i in range(n_ph)])) for a in range(3)]
    finally:
        N.nsa_set_phase_events(None)
        hev.close()
    b_keys, b_sel, b_step = dsa_bytes(case)
    flops = 2 * wl.batch * wl.num_heads * k * (wl.d_qk + wl.d_v)
    res = dict(workload=wl.name, ms_per_step=ms, tokens_per_s=wl.batch / (ms * 1e-3), step_bytes=b_step,
               gbs=b_step / (ms * 1e-3) / 1e9,
               kernel_us=dict(indexer=ph[0] * 1e3, select=ph[1] * 1e3, attention_and_combine=ph[2] * 1e3),
               indexer_gbs=b_keys / (ph[0] * 1e-3) / 1e9, attention_tflops=flops / (ph[2] * 1e-3) / 1e12,
               attention_bytes=b_sel, attention_flops=flops)
    res["hbm_frac"] = res["gbs"] / HBM_PEAK_GBS
    res["phase_clock_us"] = decode_phase_clock(torch, N, step,
                                               kernels=((0, "topk", DSA_K0_PHASES), (1, "attn", DSA_K1_PHASES)))
    log("[bench] dsa phase clock (us after the first top-k workgroup starts; median / max over workgroups): " +
        ", ".join(f"{k} {v['median_us']}/{v['max_us']}" for k, v in res["phase_clock_us"].items()))
    if not args.no_cpu:
        res["cpu"] = dsa_cpu_baseline(case, args.cpu_seconds / 2)
    log(f"[bench] dsa {wl.name}: {ms * 1e3:.1f} us/step, {res['tokens_per_s']:.4g} tok/s, {res['gbs']:.0f} GB/s "
        f"({100 * res['hbm_frac']:.1f}%); indexer {ph[0] * 1e3:.1f} us ({res['indexer_gbs']:.0f} GB/s), select "
        f"{ph[1] * 1e3:.1f} us, attention+combine {ph[2] * 1e3:.1f} us ({res['attention_tflops']:.0f} TFLOP/s)")
    return res


_POOL_CASE = None   # the case the forked oracle workers read (shared copy-on-write)


def _oracle_worker_init():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)          # one BLAS thread per worker
    except Exception:
        pass


def _oracle_pair(task):
    """One (sequence, KV group) of the decode workload: its compressed cache
    (untimed: the decode workload holds it precomputed), then the float64 decode
    query repeated until `seconds` of work.  Returns (queries, seconds, selection)."""
    from oracle import nsa_oracle as O
    b, g, seconds = task
    case = _POOL_CASE
    p = case.p
    G = case.wl.num_q_heads // case.wl.num_kv_heads
    K, V, Kc, Vc = O.compress_group(case, b, g)
    t = int(case.seq_lens[b]) - 1
    qg = O._widen(case.q[b, g * G:(g + 1) * G])
    gates = np.asarray(case.gates[b, g * G:(g + 1) * G], np.float64)
    n, el, idx = 0, 0.0, None
    while el < seconds or n == 0:
        t0 = time.perf_counter()
        r = O.nsa_query(qg, K, V, Kc, Vc, t, gates, p.l, p.d, p.l_sel, p.n_sel, p.n_local, p.force_initial, p.w)
        el += time.perf_counter() - t0
        n += 1
        idx = r.idx
    return n, el, idx


def host_info():
    """CPU model and the NumPy / BLAS build the oracle ran on."""
    model = None
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                model = ln.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    blas = None
    try:
        from threadpoolctl import threadpool_info
        blas = [{k: i.get(k) for k in ("internal_api", "version", "architecture")} for i in threadpool_info()]
    except Exception:
        pass
    return {"cpu_model": model, "numpy": np.__version__, "blas": blas}


def cpu_baseline(case, min_seconds):
    """The float64 oracle on the decode workload, on this host's cores: a pool of
    one single-threaded worker per core (of this process's affinity set, at most
    16), each taking (sequence, KV group) pairs of the workload and repeating its
    decode query for a bounded time.  Throughput = the workers' summed query
    rates / KV groups per token.  Runs before the GPU is touched (the workers are
    forked)."""
    import multiprocessing as mp
    global _POOL_CASE
    wl = case.wl
    cores = min(16, len(os.sched_getaffinity(0)))
    pairs = [(b, g) for b in range(wl.batch) for g in range(wl.num_kv_heads)]
    per_task = max(0.5, min_seconds * cores / len(pairs))
    _POOL_CASE = case
    t0 = time.perf_counter()
    with mp.get_context("fork").Pool(cores, initializer=_oracle_worker_init) as pool:
        res = pool.map(_oracle_pair, [(b, g, per_task) for b, g in pairs], chunksize=1)
    wall = time.perf_counter() - t0
    _POOL_CASE = None
    rate = sum(n / el for n, el, _ in res) / wl.num_kv_heads      # tokens/s with every worker busy
    sel = np.full((wl.batch, wl.num_kv_heads, wl.params.n_sel), -1, np.int64)
    for (b, g), (_, _, idx) in zip(pairs, res):
        sel[b, g, :len(idx)] = idx
    work = sum(el for _, el, _ in res)
    out = dict(value=rate, unit="tokens/s", cores=cores, kind="oracle",
               sample=f"every (sequence, KV group) pair of {wl.name} ({len(pairs)}), each decode query repeated for "
                      f"about {per_task:.1f} s on one of {cores} single-threaded workers ({work:.1f} s of CPU work, "
                      f"{wall:.1f} s wall including the untimed compression of each pair's cache)")
    out.update(host_info())
    return out, needle_hits(case, sel)


def dsa_cpu_baseline(case, min_seconds):
    """The float64 DSA oracle on a bounded sample of decode queries (this host's cores)."""
    from oracle import dsa_oracle as D
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = 1
    tokens, elapsed = 0, 0.0
    while elapsed < min_seconds:
        for b in range(case.wl.batch):
            t0 = time.perf_counter()
            D.decode_sequence(case, b)
            elapsed += time.perf_counter() - t0
            tokens += 1
            if elapsed >= min_seconds:
                break
    return dict(value=tokens / elapsed, unit="tokens/s", cores=int(threads), kind="oracle",
                sample=f"{tokens} DSA decode queries of {case.wl.name} (indexer over the full context, top-k, "
                       f"attention); {elapsed:.1f} s of CPU work")


def kernels_only(args, torch, N, I):
    """A few eager calls and nothing else (for profiler runs): decode steps over
    the cache copies, or, with --prefill, prefill calls."""
    if args.dsa:
        wl = I.dsa_workload("dsa_decode_64k_b8")
        case = I.generate_dsa(wl, list(I.DSA_WORKLOADS).index(wl.name))
        dims, T = dsa_upload(case, torch, N)
        ws = N.new_workspace(N.nsa_dsa_decode_workspace_size(dims, wl.top_k, wl.seq_len))
        out = torch.empty((wl.batch, wl.num_heads, wl.d_v), dtype=torch.bfloat16, device="cuda")
        copies = [(T["c"], T["ki"])] + [(T["c"].clone(), T["ki"].clone()) for _ in range(args.copies - 1)]
        for i in range(args.kernels_only):
            c, ki = copies[i % len(copies)]
            N.nsa_dsa_decode_fwd(dims, wl.top_k, T["q"], T["qi"], T["wi"], c, ki, T["seq"], wl.seq_len, out, None,
                                 ws)
        torch.cuda.synchronize()
        log(f"[bench] {args.kernels_only} DSA decode steps of {wl.name} done")
        return
    if args.backward:
        _, attn, comp, _, _ = backward_setup(torch, N, I)
        for i in range(args.kernels_only):
            attn()
            comp()
            torch.cuda.synchronize()
            log(f"[bench] backward call {i + 1}/{args.kernels_only} done")
        return
    if args.prefill:
        wl = I.workload("prefill_32k")
        case = I.generate(wl, list(I.WORKLOADS).index("prefill_32k"))
        p = wl.params

        def dev(a):
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()

        dims = N.make_dims(wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.d_k, wl.d_v)
        cfg = N.make_config(p.l, p.d, p.l_sel, p.n_sel, p.n_local, p.force_initial, p.w)
        q, k, v = dev(case.q), dev(case.k), dev(case.v)
        wk, pk, wv, pv = dev(case.w_k), dev(case.pe_k), dev(case.w_v), dev(case.pe_v)
        gates = torch.from_numpy(case.gates).cuda()
        out = torch.empty((wl.batch, wl.seq_len, wl.num_q_heads, wl.d_v), dtype=torch.bfloat16, device="cuda")
        ws = N.new_workspace(N.nsa_prefill_workspace_size(dims, cfg, wl.seq_len, True))
        for i in range(args.kernels_only):
            N.nsa_prefill_fwd(dims, cfg, wl.seq_len, q, k, v, None, None, wk, pk, wv, pv, gates, out, None, ws)
            torch.cuda.synchronize()
            log(f"[bench] prefill call {i + 1}/{args.kernels_only} done")
        return
    wl = I.workload(args.workload)
    case = I.generate(wl, list(I.WORKLOADS).index(args.workload))
    dims, cfg, T, max_len, cuc = upload_case(case, torch, N)
    ws = N.new_workspace(N.nsa_decode_workspace_size(dims, cfg, max_len))
    out = torch.empty((wl.batch, wl.num_q_heads, wl.d_v), dtype=torch.bfloat16, device="cuda")
    copies = [(T["k"], T["v"], T["kc"], T["vc"])]
    for _ in range(args.copies - 1):
        copies.append(tuple(x.clone() for x in copies[0]))
    torch.cuda.synchronize()
    ws_a = N.new_workspace(N.nsa_compress_append_workspace_size(dims, cfg)) if args.serving else None
    for i in range(args.kernels_only):
        k, v, kc, vc = copies[i % len(copies)]
        if args.serving:
            N.nsa_compress_append(dims, cfg, k, v, T["cu"], T["seq"], max_len, T["w_k"], T["pe_k"], T["w_v"],
                                  T["pe_v"], kc, vc, T["cuc"], ws_a)
        N.nsa_decode_fwd(dims, cfg, T["q"], k, v, kc, vc, T["seq"], T["cu"], T["cuc"], max_len, T["gates"], out,
                         None, ws)
    torch.cuda.synchronize()
    log(f"[bench] {args.kernels_only} {'serving' if args.serving else 'decode'} steps of {wl.name} done")


def measured_peaks(torch):
    """Peaks measured on this GPU: HBM by a 4 GiB device copy (read + write) and a
    4 GiB read-only reduction, bf16 MFMA by a large torch.matmul (hipBLASLt);
    best of several runs each."""
    n = 1 << 31  # bf16 elements = 4 GiB
    x = torch.ones(n, dtype=torch.bfloat16, device="cuda")
    y = torch.empty_like(x)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def best(fn, reps=5):
        fn()
        torch.cuda.synchronize()
        t = []
        for _ in range(reps):
            ev0.record()
            fn()
            ev1.record()
            torch.cuda.synchronize()
            t.append(ev0.elapsed_time(ev1))
        return min(t) * 1e-3

    copy_gbs = 2 * 2 * n / best(lambda: y.copy_(x)) / 1e9
    xf = x.view(torch.float32)
    read_gbs = 2 * n / best(lambda: torch.sum(xf)) / 1e9
    del x, y, xf
    m = 8192
    a = torch.randn((m, m), dtype=torch.bfloat16, device="cuda")
    b = torch.randn((m, m), dtype=torch.bfloat16, device="cuda")
    gemm = 2 * m ** 3 / best(lambda: torch.matmul(a, b), reps=10) / 1e12
    del a, b
    torch.cuda.empty_cache()
    res = {"hbm_copy_GB/s": copy_gbs, "hbm_read_GB/s": read_gbs, "bf16_gemm_TFLOP/s": gemm,
           "how": "4 GiB torch copy_ (bytes read + written) and torch.sum over the same 4 GiB (bytes read); "
                  "torch.matmul 8192^3 bf16; best of 5 / 10"}
    log(f"[bench] measured peaks: copy {copy_gbs:.0f} GB/s, read {read_gbs:.0f} GB/s, bf16 GEMM {gemm:.0f} TFLOP/s")
    return res


def copy_calibration(torch, mib=256, reps=4):
    """A plain device copy of known size (torch's copy kernel), for scaling the
    HBM byte counters of a profiler run: each launch reads and writes mib MiB."""
    n = mib * 1024 * 1024 // 2
    x = torch.ones(n, dtype=torch.bfloat16, device="cuda")
    y = torch.empty_like(x)
    for _ in range(reps):
        y.copy_(x)
    torch.cuda.synchronize()
    log(f"[bench] copy calibration: {reps} copies of {mib} MiB done")


TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "decode_stream_kernel.decode_64k_b8.traffic.md")


def roofline_from_profiles(kernel_hash):
    """HBM bytes per launch of the streaming kernel from the committed rocprofv3
    counter summary (FETCH_SIZE and WRITE_SIZE scaled by a plain copy of known
    size), or None when that summary was taken on other kernel sources."""
    try:
        fields = {}
        for ln in open(TRAFFIC_PROFILE):
            if ":" in ln and ln.strip().startswith("- "):
                k, v = ln.strip()[2:].split(":", 1)
                fields[k.strip()] = v.strip().strip("`")
        if fields.get("kernel_src_hash") == kernel_hash:
            return int(fields["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        pass
    return None


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=60)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="decode_64k_b8")
    ap.add_argument("--copies", type=int, default=6)
    ap.add_argument("--prefill-reps", type=int, default=3)
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-configs", action="store_true", help="skip the 128k and ragged decode workloads")
    ap.add_argument("--no-serving", action="store_true", help="skip the append + decode serving-step timing")
    ap.add_argument("--no-dsa", action="store_true", help="skip the DSA decode workload")
    ap.add_argument("--dsa", action="store_true", help="with --kernels-only: DSA decode steps")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--kernels-only", type=int, default=0, metavar="N",
                    help="run N eager calls and exit (for profiler runs; no timing, no JSON line)")
    ap.add_argument("--prefill", action="store_true", help="with --kernels-only: prefill calls instead of decode")
    ap.add_argument("--backward", action="store_true",
                    help="with --kernels-only: prefill backward calls (attention and compression)")
    ap.add_argument("--no-backward", action="store_true", help="skip the prefill backward")
    ap.add_argument("--serving", action="store_true",
                    help="with --kernels-only: nsa_compress_append before every decode call")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run a plain 256 MiB device copy a few times and exit (profiler counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this NSA path is single-GPU by design; run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import long_context_sparse_nsa_amd as N
    import nsa_inputs as I
    N.load_library()
    if args.copy_calibration or args.kernels_only:
        torch.cuda.set_device(0)
        if args.copy_calibration:
            copy_calibration(torch)
        else:
            kernels_only(args, torch, N, I)
        return

    # the headline workload's inputs, and the float64 oracle on this host's cores
    # (forked workers: before anything touches the GPU)
    wl = I.workload(args.workload)
    t0 = time.time()
    case = I.generate(wl, list(I.WORKLOADS).index(args.workload))
    log(f"[bench] generated {wl.name} in {time.time() - t0:.1f}s")
    cpu, needle_oracle = (None, None) if args.no_cpu else cpu_baseline(case, args.cpu_seconds)
    if cpu:
        log(f"[bench] cpu oracle: {cpu['value']:.3g} tok/s on {cpu['cores']} single-threaded workers "
            f"({cpu['cpu_model']}); oracle needle-hit rate {needle_oracle}")

    torch.cuda.set_device(0)
    peaks = measured_peaks(torch)
    case, dec, _ = bench_decode(args, torch, N, I, args.workload, case=case, headline=True)
    others = {}
    if not args.no_configs:
        for name in ("decode_128k_b4", "decode_ragged_16"):
            if name != args.workload:
                others[name] = bench_decode(args, torch, N, I, name)[1]
                torch.cuda.empty_cache()
    pre = None if args.no_prefill else bench_prefill(args, torch, N, I)
    bwd = None if args.no_backward else bench_backward(args, torch, N, I)
    dsa = None if args.no_dsa else bench_dsa(args, torch, N, I)

    khash = src_hash(*DECODE_SOURCES)
    p = wl.params

    def decode_entry(d):
        return {"ms_per_step": d["ms_per_step"], "tokens_per_s": d["tokens_per_s"],
                "warm_ms_per_step": d["warm_ms_per_step"], "step_distribution": d["step_distribution"],
                "algorithmic_bytes": d["step_bytes"], "GB/s": d["step_gbs"], "hbm_frac": d["step_frac"],
                "hbm_frac_of_measured_copy": d["step_gbs"] / peaks["hbm_copy_GB/s"],
                "kernel_us": {"decode_stream_kernel": d["pass1_us"], "decode_finish_kernel": d["finish_us"]},
                "needle_hit_rate_gpu": d["needle_hit_gpu"]}

    line = {
        "metric": METRIC,
        "value": dec["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": dec["steps"],
        "warmup": args.warmup,
        "ms_per_step": dec["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": wl.batch, "context": wl.seq_len, "q_heads": wl.num_q_heads,
                   "kv_heads": wl.num_kv_heads, "d_k": wl.d_k, "d_v": wl.d_v, "l": p.l, "d": p.d,
                   "l_sel": p.l_sel, "n_sel": p.n_sel, "w": p.w, "timing": dec["timing"],
                   "cache_copies": args.copies},
        "roofline": {"bound": "hbm", "kernel": "decode_stream_kernel (compressed branch, folded scores, window)",
                     "achieved": dec["pass1_gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": dec["pass1_gbs"] / HBM_PEAK_GBS, "traffic": roofline_from_profiles(khash),
                     "duration_us": dec["pass1_us"], "algorithmic_bytes": dec["pass1_bytes"],
                     "frac_of_measured_copy": dec["pass1_gbs"] / peaks["hbm_copy_GB/s"],
                     "step": {"achieved": dec["step_gbs"], "frac": dec["step_frac"],
                              "frac_of_measured_copy": dec["step_gbs"] / peaks["hbm_copy_GB/s"],
                              "algorithmic_bytes": dec["step_bytes"], "duration_us": dec["ms_per_step"] * 1e3}},
        "decode_step": dict(decode_entry(dec), wall_s_timed_region=dec["wall_s"],
                            phase_clock_us=dec.get("phase_clock_us"), needle_hit_rate_oracle=needle_oracle),
        "decode_configs": {k: decode_entry(v) for k, v in others.items()},
        "measured_peaks": peaks,
        "cpu_baseline": cpu,
    }
    line["gate_network"] = {
        "reading": "gate[h, c] = sigmoid(w_gate[h, c] . q[h] + b_gate[h, c]), computed in the kernels that apply it",
        "decode_ms_per_step": dec.get("gate_network_ms_per_step"),
        "prefill_ms": pre.get("gate_network_ms") if pre else None}
    if dsa:
        line["dsa_decode"] = {
            "workload": dsa["workload"], "ms_per_step": dsa["ms_per_step"], "tokens_per_s": dsa["tokens_per_s"],
            "algorithmic_bytes": dsa["step_bytes"], "GB/s": dsa["gbs"], "hbm_frac": dsa["hbm_frac"],
            "kernel_us": dsa["kernel_us"],
            "indexer": {"kernel": "dsa_index_kernel", "bound": "hbm", "GB/s": dsa["indexer_gbs"],
                        "frac": dsa["indexer_gbs"] / HBM_PEAK_GBS},
            "attention": {"kernels": "dsa_attn_kernel + dsa_combine_kernel", "TFLOP/s": dsa["attention_tflops"],
                          "mfma_frac": dsa["attention_tflops"] / MFMA_BF16_PEAK_TFLOPS},
            "phase_clock_us": dsa.get("phase_clock_us"),
            "cpu_oracle": dsa.get("cpu")}
    if dec.get("serving"):
        sv = dec["serving"]
        line["serving_step"] = {
            "calls": "nsa_compress_append + nsa_decode_fwd", "ms_per_step": sv["ms_per_step"],
            "tokens_per_s": sv["tokens_per_s"],
            "append": {"kernels": "append_partial_kernel + append_reduce_kernel", "us": sv["append_us"],
                       "blocks": sv["append_rows"], "algorithmic_bytes": sv["append_bytes"],
                       "GB/s": sv["append_gbs"], "hbm_frac": sv["append_hbm_frac"]}}
    if pre:
        line["prefill"] = {"workload": pre["workload"], "ms": pre["ms"], "TFLOP/s": pre["tflops"],
                           "mfma_frac": pre["mfma_frac"], "flops": pre["flops"],
                           "peak_TFLOP/s": MFMA_BF16_PEAK_TFLOPS, "kernel_ms": pre["kernel_ms"],
                           "mfma_frac_of_measured_gemm": pre["tflops"] / peaks["bf16_gemm_TFLOP/s"],
                           "selected_branch": {"kernel": "pf_sel_kernel", "TFLOP/s": pre["sel_tflops"],
                                               "mfma_frac": pre["sel_mfma_frac"],
                                               "mfma_frac_of_measured_gemm":
                                                   pre["sel_tflops"] / peaks["bf16_gemm_TFLOP/s"],
                                               "reuse": pre["selected_reuse"]},
                           "cmp_win_topn": {"kernel": "pf_cmp_win_kernel", "TFLOP/s": pre["cmp_win_tflops"],
                                            "mfma_frac": pre["cmp_win_tflops"] / MFMA_BF16_PEAK_TFLOPS}}
    if bwd:
        line["prefill_backward"] = {
            "workload": bwd["workload"], "calls": "nsa_prefill_bwd + nsa_compress_bwd (keys, values)",
            "ms": bwd["ms"], "TFLOP/s": bwd["tflops"], "flops": bwd["flops"],
            "attention": {"ms": bwd["attention_ms"], "TFLOP/s": bwd["attention_tflops"],
                          "mfma_frac": bwd["mfma_frac"], "peak_TFLOP/s": MFMA_BF16_PEAK_TFLOPS,
                          "kernel_ms": bwd["kernel_ms"]},
            "compression_ms": bwd["compress_ms"], "positions_per_s": bwd["positions_per_s"],
            "attention_ms_without_saved_lse": bwd["recompute_ms"],
            "cpu_oracle": bwd.get("cpu")}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
