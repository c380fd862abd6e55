"""GPU parity of the in-kernel gate network (sigmoid of one linear layer of each
query head) in decode and prefill against the float64 oracle."""
import numpy as np
import pytest

import nsa_inputs as I
from tests import gpu_util as U
from tests.test_gpu_decode import _check_decode
from tests.test_gpu_prefill import _check_rows

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("bias", [True, False])
def test_decode_gate_network(bias):
    case = I.generate(I.workload("decode_64k_b8", batch=3, seq_len=6000, ragged_min=2500), 41)
    case.gate_net = True
    if not bias:
        case.b_gate = None
    kc, vc, _ = U.oracle_cmp_cache(case)
    out, sel, _ = U.run_decode(case, kc, vc)
    _check_decode(case, out, sel)


def test_decode_gate_network_small_group():
    """Four query heads per KV head, d_k = d_v = 64."""
    case = I.generate(I.workload("decode_64k_b8", batch=2, seq_len=3000, num_q_heads=8, num_kv_heads=2,
                                 d_k=64, d_v=64), 42)
    case.gate_net = True
    kc, vc, _ = U.oracle_cmp_cache(case)
    out, sel, _ = U.run_decode(case, kc, vc)
    _check_decode(case, out, sel)


def test_decode_gate_network_saturated_gates():
    """Large pre-activations: gates at 0 and 1 exactly isolate branches."""
    case = I.generate(I.workload("decode_64k_b8", batch=2, seq_len=4000), 43)
    case.gate_net = True
    case.w_gate = np.zeros_like(case.w_gate)  # bf16 zeros
    case.b_gate = np.tile(np.array([-60.0, 60.0, -60.0], np.float32), (case.wl.num_q_heads, 1))
    kc, vc, _ = U.oracle_cmp_cache(case)
    out, sel, _ = U.run_decode(case, kc, vc)
    _check_decode(case, out, sel)


def test_tiny_prefill_gate_network():
    case = I.generate(I.workload("tiny_prefill_512"), 44)
    case.gate_net = True
    out, sel = U.run_prefill(case)
    _check_rows(case, out, sel, range(512))


def test_prefill_gate_network_wide_heads():
    """d_k = 192, 16 heads per group, a ragged last tile."""
    case = I.generate(I.workload("prefill_32k", seq_len=1100), 45)
    case.gate_net = True
    out, sel = U.run_prefill(case)
    _check_rows(case, out, sel, range(1100))
