"""Host-only checks of the C ABI: the library loads, exports what include/nsa.h
declares, and rejects invalid arguments before anything reaches the GPU."""
import ctypes
import os
import re

import pytest

import long_context_sparse_nsa_amd as N
from long_context_sparse_nsa_amd import _abi as A

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nsa.h")

lib_missing = not os.path.exists(A.lib_path())
pytestmark = pytest.mark.skipif(lib_missing, reason="libnsa.so not built (run __graft_entry__.build())")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(nsa_[a-z_]+)\s*\(", src)))


def test_header_declares_the_entry_points():
    fns = declared_functions()
    for name in ("nsa_compress_kv", "nsa_prefill_fwd", "nsa_decode_fwd", "nsa_decode_workspace_size",
                 "nsa_prefill_workspace_size", "nsa_status_string", "nsa_last_error"):
        assert name in fns


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(A.lib_path())
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert set(declared_functions()) == set(A.EXPORTS)


def test_status_strings():
    assert N.nsa_status_string(0) == "NSA_SUCCESS"
    assert N.nsa_status_string(3) == "NSA_ERROR_WORKSPACE"


STD = dict(l=32, d=16, l_sel=64, n_sel=16, n_local=2, force_initial=1, w=512)


def _cfg(**kw):
    a = dict(STD)
    a.update(kw)
    return N.make_config(**a)


def _dims(**kw):
    a = dict(batch=8, num_q_heads=64, num_kv_heads=4, d_k=192, d_v=128)
    a.update(kw)
    return N.make_dims(**a)


def _ws(dims, cfg, L=65536):
    return N.nsa_decode_workspace_size(dims, cfg, L)


def test_workspace_sizes_are_positive_and_monotone():
    a = _ws(_dims(), _cfg(), 4096)
    b = _ws(_dims(), _cfg(), 65536)
    c = _ws(_dims(batch=16), _cfg(), 65536)
    assert 0 < a < b < c
    # prefill: fp32 partial output [T, 64, 128] + selection ids [T, 4, 16], plus the
    # compressed cache when compressing in the call
    base = 32768 * 64 * 128 * 4 + 32768 * 4 * 16 * 4
    assert N.nsa_prefill_workspace_size(_dims(batch=1), _cfg(), 32768, False) == base
    assert N.nsa_prefill_workspace_size(_dims(batch=1), _cfg(), 32768, True) >= base + 4 * 2047 * (192 + 128) * 2
    assert N.nsa_prefill_workspace_size(_dims(batch=1), _cfg(), 65536, False) > 0   # 1024 blocks: supported


@pytest.mark.parametrize("dims_kw,cfg_kw,L,status", [
    (dict(num_q_heads=63), {}, 100, A.NSA_ERROR_INVALID_VALUE),
    (dict(batch=0), {}, 100, A.NSA_ERROR_INVALID_VALUE),
    (dict(d_k=100), {}, 100, A.NSA_ERROR_UNSUPPORTED),
    (dict(num_q_heads=128), {}, 100, A.NSA_ERROR_UNSUPPORTED),        # group of 32 heads
    ({}, dict(d=0), 100, A.NSA_ERROR_INVALID_VALUE),
    ({}, dict(force_initial=2), 100, A.NSA_ERROR_INVALID_VALUE),
    ({}, dict(l=24), 100, A.NSA_ERROR_UNSUPPORTED),                    # l_sel/d=4 ok, d does not divide l? 24%16
    ({}, dict(l=128), 100, A.NSA_ERROR_UNSUPPORTED),                   # l > l_sel
    ({}, dict(l_sel=48, d=16), 100, A.NSA_ERROR_UNSUPPORTED),          # l_sel/d = 3
    ({}, dict(n_sel=65), 100, A.NSA_ERROR_UNSUPPORTED),
    ({}, dict(n_sel=2, n_local=2), 100, A.NSA_ERROR_UNSUPPORTED),      # forced blocks exceed n
    ({}, {}, 0, A.NSA_ERROR_INVALID_VALUE),
    ({}, {}, 64 * 8192 + 1, A.NSA_ERROR_UNSUPPORTED),                  # too many selection blocks
])
def test_validation_errors(dims_kw, cfg_kw, L, status):
    with pytest.raises(N.NSAError) as e:
        _ws(_dims(**dims_kw), _cfg(**cfg_kw), L)
    assert e.value.status == status
    assert N.nsa_last_error() != ""


def _raw_decode(dims, cfg, ptr, L, ws, ws_bytes):
    lib = A.load_library()
    return lib.nsa_decode_fwd(ctypes.byref(dims), ctypes.byref(cfg), ptr, ptr, ptr, ptr, ptr, ptr, None, None,
                              L, ptr, None, None, ptr, None, ws, ws_bytes, None)


def test_decode_rejects_null_tensor_and_small_workspace_without_launching():
    dims, cfg = _dims(), _cfg()
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first
    lib = A.load_library()
    st = lib.nsa_decode_fwd(ctypes.byref(dims), ctypes.byref(cfg), None, fake, fake, fake, fake, fake, None, None,
                            65536, fake, None, None, fake, None, fake, 1 << 30, None)
    assert st == A.NSA_ERROR_INVALID_VALUE and "NULL" in N.nsa_last_error()
    # gate sources: none, or both given values and the gate network
    for gates, wg, bgt in ((None, None, None), (fake, fake, None), (fake, None, fake)):
        st = lib.nsa_decode_fwd(ctypes.byref(dims), ctypes.byref(cfg), fake, fake, fake, fake, fake, fake, None,
                                None, 65536, gates, wg, bgt, fake, None, fake, 1 << 30, None)
        assert st == A.NSA_ERROR_INVALID_VALUE and "gate" in N.nsa_last_error()
    need = _ws(dims, cfg, 65536)
    assert _raw_decode(dims, cfg, fake, 65536, fake, need - 1) == A.NSA_ERROR_WORKSPACE
    assert _raw_decode(dims, cfg, fake, 65536, None, need) == A.NSA_ERROR_WORKSPACE
    assert str(need) in N.nsa_last_error()


def test_prefill_rejects_half_given_cache_and_missing_weights():
    lib = A.load_library()
    dims, cfg = _dims(batch=1), _cfg()
    f = ctypes.c_void_p(0x1000)
    st = lib.nsa_prefill_fwd(ctypes.byref(dims), ctypes.byref(cfg), 4096, f, f, f, f, None, f, f, f, f, f, None, None,
                             f, None, None, f, 1 << 30, None)
    assert st == A.NSA_ERROR_INVALID_VALUE
    st = lib.nsa_prefill_fwd(ctypes.byref(dims), ctypes.byref(cfg), 4096, f, f, f, None, None, None, f, f, f, f, None,
                             None, f, None, None, f, 1 << 30, None)
    assert st == A.NSA_ERROR_INVALID_VALUE
    st = lib.nsa_prefill_fwd(ctypes.byref(dims), ctypes.byref(cfg), 70000, f, f, f, f, f, None, None, None, None, f,
                             None, None, f, None, None, None, 0, None)
    assert st == A.NSA_ERROR_UNSUPPORTED


def test_append_workspace_size_and_validation():
    # fp32 partials: max(ceil(32*192/256), ceil(32*128/256)) = 24 chunks x 64 padded rows x 320 channels
    assert N.nsa_compress_append_workspace_size(_dims(), _cfg()) == 24 * 64 * 320 * 4
    assert N.nsa_compress_append_workspace_size(_dims(batch=17), _cfg()) == 24 * 128 * 320 * 4
    lib = A.load_library()
    dims, cfg = _dims(), _cfg()
    f = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first
    need = N.nsa_compress_append_workspace_size(dims, cfg)

    def call(seq_lens, ws, ws_bytes, max_len=65536):
        return lib.nsa_compress_append(ctypes.byref(dims), ctypes.byref(cfg), f, f, None, seq_lens, max_len, f, f, f,
                                       f, f, f, None, ws, ws_bytes, None)
    assert call(None, f, need) == A.NSA_ERROR_INVALID_VALUE and "NULL" in N.nsa_last_error()
    assert call(f, f, need - 1) == A.NSA_ERROR_WORKSPACE
    assert call(f, None, need) == A.NSA_ERROR_WORKSPACE
    assert call(f, f, need, max_len=0) == A.NSA_ERROR_INVALID_VALUE
    bad = _cfg(l_sel=48)
    assert lib.nsa_compress_append(ctypes.byref(dims), ctypes.byref(bad), f, f, None, f, 100, f, f, f, f, f, f, None,
                                   f, need, None) == A.NSA_ERROR_UNSUPPORTED


def _dsa_dims(**kw):
    a = dict(batch=8, num_heads=128, d_qk=576, d_v=512, idx_heads=16, idx_dim=128)
    a.update(kw)
    return N.make_dsa_dims(**a)


def test_dsa_workspace_and_validation():
    ws = N.nsa_dsa_decode_workspace_size(_dsa_dims(), 2048, 65536)
    # at least the fp32 scores and the selection buffer
    assert ws >= 8 * 65536 * 4 + 8 * 2048 * 4
    assert N.nsa_dsa_decode_workspace_size(_dsa_dims(batch=1), 2048, 4096) < ws
    for kw, k, L, status in [
        (dict(d_qk=512), 2048, 4096, A.NSA_ERROR_UNSUPPORTED),
        (dict(num_heads=48), 2048, 4096, A.NSA_ERROR_UNSUPPORTED),
        (dict(idx_heads=8), 2048, 4096, A.NSA_ERROR_UNSUPPORTED),
        (dict(idx_dim=96), 2048, 4096, A.NSA_ERROR_UNSUPPORTED),
        ({}, 4097, 4096, A.NSA_ERROR_UNSUPPORTED),
        ({}, 2048, 65537, A.NSA_ERROR_UNSUPPORTED),
        ({}, 0, 4096, A.NSA_ERROR_INVALID_VALUE),
        (dict(batch=0), 2048, 4096, A.NSA_ERROR_INVALID_VALUE),
    ]:
        with pytest.raises(N.NSAError) as e:
            N.nsa_dsa_decode_workspace_size(_dsa_dims(**kw), k, L)
        assert e.value.status == status
    lib = A.load_library()
    d = _dsa_dims()
    f = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first
    need = N.nsa_dsa_decode_workspace_size(d, 2048, 65536)
    call = lambda q, ws, nb: lib.nsa_dsa_decode_fwd(ctypes.byref(d), 2048, 0.0, q, f, f, f, f, f, 65536, f, None, ws,
                                                    nb, None)
    assert call(None, f, need) == A.NSA_ERROR_INVALID_VALUE and "NULL" in N.nsa_last_error()
    assert call(f, f, need - 1) == A.NSA_ERROR_WORKSPACE
    assert call(f, None, need) == A.NSA_ERROR_WORKSPACE


def test_null_dims_and_config():
    lib = A.load_library()
    out = ctypes.c_size_t(0)
    assert lib.nsa_decode_workspace_size(None, ctypes.byref(_cfg()), 100, ctypes.byref(out)) == A.NSA_ERROR_INVALID_VALUE
    assert lib.nsa_decode_workspace_size(ctypes.byref(_dims()), None, 100, ctypes.byref(out)) == A.NSA_ERROR_INVALID_VALUE


def test_binding_refuses_host_tensors():
    import torch
    with pytest.raises(ValueError):
        A._ptr(torch.zeros(4), "x")


def test_backward_workspace_sizes_and_validation():
    dims, cfg = _dims(batch=1), _cfg()
    T = 32768
    # statistics records [3, 1, T, 4, 48] fp32, bitmap [1, 4, T/64, T/32] uint32, selected-branch
    # partials [4, slots, 64, 320] fp32, compressed-branch partials [32, 1, 4, nc, 320] fp32 (ranges
    # of 1024 positions), tile counts and slot offsets int32, gate-gradient partials [64, 64, 3, 193]
    nc = (T - 32) // 16 + 1
    r256 = lambda x: -(-x // 256) * 256
    slots = 512 + T * 16 // 512  # key tiles + positions x n_sel / 512
    assert N.nsa_prefill_bwd_workspace_size(dims, cfg, T) == (3 * T * 4 * 48 * 4 + 4 * 512 * 1024 * 4 +
                                                             4 * slots * 64 * 320 * 4 + r256(32 * 4 * nc * 320 * 4) +
                                                             r256(4 * 512 * 4) + r256(4 * 513 * 4) +
                                                             r256(64 * 64 * 3 * 193 * 4))
    assert N.nsa_compress_bwd_workspace_size(dims, cfg, T, 0) == 64 * 192 * 4 + 8 * 32 * 192 * 192 * 4
    assert N.nsa_compress_bwd_workspace_size(dims, cfg, T, 1) == 64 * 128 * 4 + 8 * 32 * 128 * 128 * 4
    lib = A.load_library()
    f = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first
    need = N.nsa_prefill_bwd_workspace_size(dims, cfg, T)

    def bwd(q=f, kc=f, sel=f, ws=f, nb=need, T=T, gates=f, wg=None, bg=None, dwg=None):
        return lib.nsa_prefill_bwd(ctypes.byref(dims), ctypes.byref(cfg), T, q, f, f, kc, f, gates, wg, bg, sel, None,
                                   f, f, f, f, f, f, f, dwg, None, ws, nb, None)
    assert bwd(q=None) == A.NSA_ERROR_INVALID_VALUE and "NULL" in N.nsa_last_error()
    assert bwd(sel=None) == A.NSA_ERROR_INVALID_VALUE
    assert bwd(kc=None) == A.NSA_ERROR_INVALID_VALUE and "compressed" in N.nsa_last_error()
    assert bwd(nb=need - 1) == A.NSA_ERROR_WORKSPACE
    assert bwd(ws=None) == A.NSA_ERROR_WORKSPACE
    assert bwd(T=0) == A.NSA_ERROR_INVALID_VALUE
    assert bwd(T=70000) == A.NSA_ERROR_UNSUPPORTED  # more than 1024 selection blocks
    assert bwd(gates=None) == A.NSA_ERROR_INVALID_VALUE  # no gate source
    assert bwd(wg=f, dwg=f) == A.NSA_ERROR_INVALID_VALUE  # two gate sources
    assert bwd(gates=None, wg=f) == A.NSA_ERROR_INVALID_VALUE and "dw_gate" in N.nsa_last_error()
    assert bwd(gates=None, wg=f, bg=f, dwg=f) == A.NSA_ERROR_INVALID_VALUE  # b_gate without db_gate
    cneed = N.nsa_compress_bwd_workspace_size(dims, cfg, T, 0)

    def cbwd(which=0, x=f, dy=f, ws=f, nb=cneed):
        return lib.nsa_compress_bwd(ctypes.byref(dims), ctypes.byref(cfg), T, which, x, f, f, dy, f, f, f, ws, nb,
                                    None)
    assert cbwd(which=2) == A.NSA_ERROR_INVALID_VALUE
    assert cbwd(x=None) == A.NSA_ERROR_INVALID_VALUE
    assert cbwd(dy=None) == A.NSA_ERROR_INVALID_VALUE
    assert cbwd(nb=cneed - 1) == A.NSA_ERROR_WORKSPACE


def test_missing_library_raises_instead_of_falling_back(monkeypatch, tmp_path):
    """Without the built HIP library every entry point fails loudly: there is no
    CPU path to fall back on."""
    monkeypatch.setattr(A, "_LIB", None)
    monkeypatch.setattr(A, "lib_path", lambda: str(tmp_path / "libnsa_absent.so"))
    with pytest.raises(RuntimeError, match="not found"):
        A.load_library()
    with pytest.raises(RuntimeError, match="not found"):
        N.nsa_decode_workspace_size(_dims(), _cfg(), 512)


def test_decode_noalloc_rejects_steps_beyond_its_scratch():
    """The allocation-free decode entry point checks everything nsa_decode_fwd checks
    and refuses, before any HIP call, a step whose workspace exceeds its 32 MiB array."""
    lib = A.load_library()
    f = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first
    cfg = _cfg()
    big = _dims(batch=64)
    assert _ws(big, cfg) > 32 << 20 >= _ws(_dims(), cfg)

    def call(dims, q=f, gates=f, L=65536):
        return lib.nsa_decode_fwd_noalloc(ctypes.byref(dims), ctypes.byref(cfg), q, f, f, f, f, f, None, None, L,
                                          gates, None, None, f, None, None)
    assert call(big) == A.NSA_ERROR_UNSUPPORTED
    msg = N.nsa_last_error()
    assert "allocation-free" in msg and str(_ws(big, cfg)) in msg
    assert call(_dims(), q=None) == A.NSA_ERROR_INVALID_VALUE
    assert call(_dims(), gates=None) == A.NSA_ERROR_INVALID_VALUE
    assert call(_dims(d_k=100)) == A.NSA_ERROR_UNSUPPORTED
