"""CPU oracle for the RT-Lynx online 2:4 activation-sparse linear layer.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or
links anything here: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library (no kernels, headers, helpers, tables or generators) and imports
nothing from it.

Plain NumPy, float64 for every floating-point step, no blocking or fusion
beyond what the method's definition states.  Every function below is pinned
by ``tests/test_oracle_pins.py`` against brute force, invariants, closed
forms or library routines; none is "parity unpinned".
"""
from .rtlynx_ref import (  # noqa: F401
    bf16_bits_to_f64,
    magnitude_keys,
    select_2of4,
    brute_force_select_2of4,
    exact_magnitudes,
    l1_stats,
    compensation_scale,
    sparsify,
    compress,
    decompress,
    dense_linear_ref,
    sparse_linear_ref,
    sparse_linear_gather_ref,
    lora_down_ref,
    compressed_linear_ref,
    round_to_bf16,
    group_compensation_scale,
    sparsify_variant,
    sparse_linear_variant_ref,
)
