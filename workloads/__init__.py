"""Seeded synthetic workloads shaped like the KV caches of the PolyKV evaluation.

This package holds workload shapes and seeded random-number draws only. It holds
none of the method's arithmetic (no quantisation, rotation or attention), so that
both the CPU oracle and the HIP path can take their inputs from it without
sharing any code with each other.
"""

from .configs import CONFIGS, Config, config_by_name  # noqa: F401
from .inputs import gen_k_layer, gen_v_layer, gen_q_step, gen_k, gen_v  # noqa: F401
