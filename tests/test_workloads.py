"""The seeded generators: shapes, determinism and the intended distributions."""

import numpy as np

from workloads import CONFIGS, gen_k_layer, gen_q_step, gen_v_layer
from workloads.inputs import k_channel_scales


def test_shapes_and_dtypes():
    c = CONFIGS[0]
    k, v, q = gen_k_layer(c, 0), gen_v_layer(c, 0), gen_q_step(c, 0)
    assert k.shape == (2, 600, 128) and k.dtype == np.float16
    assert v.shape == (2, 600, 128) and v.dtype == np.float16
    assert q.shape == (1, 1, 2, 128) and q.dtype == np.float32


def test_deterministic_and_independent():
    c = CONFIGS[1]
    assert np.array_equal(gen_k_layer(c, 3), gen_k_layer(c, 3))
    assert not np.array_equal(gen_k_layer(c, 3)[0], gen_k_layer(c, 4)[0])
    assert not np.array_equal(gen_q_step(c, 0), gen_q_step(c, 1))


def test_outlier_channels():
    c = CONFIGS[2]
    s = k_channel_scales(c, 0)
    k = gen_k_layer(c, 0).astype(np.float32)
    for h in range(c.n_kv_heads):
        std = k[h].std(axis=0)
        top2 = set(np.argsort(s[h])[-2:])
        assert set(np.argsort(std)[-2:]) == top2


def test_student_t_tails():
    c = CONFIGS[4]
    v = gen_v_layer(c, 0)[:2].astype(np.float64)
    assert abs(v.var() - 2.0) < 0.15
    assert np.mean(np.abs(v) > 6) > 1e-3
