"""Plain, slow, fp64 CPU oracle of the late-layer cache fill.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
link anything under ``oracle/``: only the tests, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with
the HIP library (``late_layer_kv_amd``); its only shared dependency is the
seeded input generator ``workloads``, which holds none of the method's
arithmetic.

Every function follows a passage of "RidgeFill: Training-Free Late-Layer
Cache Fill for Faster Prefill" (arXiv 2611.09709) and says which.  The fill is
a plain definition (a map product, a normalisation, two projections, a
rotation), so the oracle is that definition written out in float64 with numpy
primitives, with no blocking, fusion or reordering.

Pins (tests/test_oracle_pins.py, run with ``-m "not gpu"``) tie every function
to something other than itself: closed forms, invariants, a library routine
the step reduces to (complex multiplication, SVD), brute-force loops on tiny
inputs and the values the pages print for the compute ceiling.  A mutation
test plants plausible mistakes in copies of these functions and checks that
some pin fails for each.  No function here is "parity unpinned".
"""
from .fill import (  # noqa: F401
    bf16_bits_to_f64, fill_row_set, predicted_input, rms_norm, project,
    rope_inv_freq, rope, layer_kv, fill_layer, fill_workload, exact_kv_workload,
    map_matrix, qk_norm, indexer_keys, fill_indexer_workload, exact_indexer_workload,
)
from .ridge import RidgeSums, ridge_fit, ridge_fit_raw  # noqa: F401
from .ceiling import layer_ceiling, mac_ceiling  # noqa: F401
from .rescale import (  # noqa: F401
    calibration_rows, fill_workload_rescaled, head_norms, rescale_values, scales_from_values, value_scales,
)
from .quant import (  # noqa: F401
    dequantize_q8, dequantize_q8_bf16, f64_to_bf16_bits, map_bytes, quantize_q8,
)
