"""Seeded synthetic inputs shared by the tests, the benchmark and the smoke
check. Holds no arithmetic of the method itself."""
from .workloads import (WORKLOADS, LayerInputs, make_layer, extra_weight, workload_layer,  # noqa: F401
                        round_to_bf16_bits, bf16_bits_to_f32, rng_for, random_codes)
