"""PolyKV oracle: a plain, slow, obviously correct CPU implementation.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package. The
library (``agent_q8_quant_amd``) never imports it, and it imports nothing from the
library: the two share no code, tables or constants.

Source of the method: "PolyKV: A Shared Asymmetrically-Compressed KV Cache Pool for
Multi-Agent LLM Inference", section "Abstract (arXiv)" (cited below as "PolyKV,
Abstract"). The abstract says that N agents share one KV pool written once, that keys
are quantised at int8 (q8_0) and that values are compressed with TurboQuant MSE: a
Fast Walsh-Hadamard Transform rotation followed by 3-bit Lloyd-Max quantisation with
centroids tuned to N(0,1). It fixes nothing finer. The finer definitions used here
(q8_0 blocks of 32 along head_dim with an fp16 absmax/127 scale and round-half-even
codes; L2 normalisation, scaling by sqrt(d) and an orthonormal Sylvester-ordered FWHT
for values; codes as counts of boundaries exceeded; a 3-plane bit layout over groups of
32 tokens) are this implementation's definitions of the open steps.

Precision: floating point is fp64 unless a step is fixed to another precision (the
q8_0 scale and quotient are float32 by definition). Every function cites the passage
it follows.

Pins. Every function here is checked by ``tests/test_oracle_*.py`` against something
other than itself: closed forms, textbook values, brute force and invariants. No
function is "parity unpinned", except the pages' 19.8 GB figure, which no function
reproduces (see ``pool.PAGES_MEMORY_FIGURES``).
"""

from .codebook import lloyd_max_gaussian, codebook_fp32, quantizer_mse_gaussian  # noqa: F401
from .hadamard import fwht, hadamard_matrix  # noqa: F401
from .q8_0 import q8_0_encode, q8_0_decode  # noqa: F401
from .turboquant import tq_mse_encode, tq_mse_decode, rotated_coordinates  # noqa: F401
from .pool import (pack_v_planes, unpack_v_planes, analytic_pool_bytes,  # noqa: F401
                   compress_pool, dequant_pool, dequant_fp16, append_pool)
from .attention import (attention_lse, attention_rows, attention_weights, pool_and_tail_decode,  # noqa: F401
                        shared_pool_decode, shared_pool_lse)
from .project import project_fp16, project_fp64  # noqa: F401
