"""MI355X (gfx950) Native Sparse Attention: forward and backward passes.

The compute lives in libnsa.so (hand-written HIP kernels behind the C ABI of
include/nsa.h); this package only marshals torch tensors into that ABI.
"""
from ._abi import (  # noqa: F401
    EXPORTS,
    NSAError,
    compressed_count,
    lib_path,
    load_library,
    make_config,
    make_dims,
    new_workspace,
    nsa_compress_append,
    nsa_compress_append_workspace_size,
    nsa_compress_bwd,
    nsa_compress_bwd_workspace_size,
    nsa_compress_kv,
    nsa_config_t,
    make_dsa_dims,
    nsa_decode_fwd,
    nsa_decode_fwd_noalloc,
    nsa_dsa_decode_fwd,
    nsa_dsa_decode_workspace_size,
    nsa_dsa_dims_t,
    nsa_decode_workspace_size,
    nsa_dims_t,
    nsa_last_error,
    nsa_prefill_bwd,
    nsa_prefill_bwd_workspace_size,
    nsa_prefill_fwd,
    nsa_prefill_workspace_size,
    nsa_set_phase_clock,
    nsa_set_phase_events,
    nsa_status_string,
)

__all__ = [n for n in dir() if n.startswith("nsa_")] + ["NSAError", "load_library", "make_config", "make_dims",
                                                        "make_dsa_dims",
                                                        "new_workspace", "compressed_count", "EXPORTS"]
