"""Seeded synthetic input generators shared by the tests, the smoke check and
the benchmark.  Holds random data only, none of the method's arithmetic."""
from .workloads import (CANARY, DTYPES, ELEM_BYTES, WORKLOADS, CacheArrays, CacheSpec,
                        StepInputs, flush_counts, make_cache, make_params, make_step,
                        random_state_bytes, tiled_index)
