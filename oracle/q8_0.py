"""q8_0 key quantisation.

PolyKV, Abstract: keys are kept at int8 in the q8_0 format, chosen there so that the
softmax stays stable.
Definition used (the pages fix nothing finer):
- blocks of 32 consecutive entries along head_dim;
- scale s = fp16(amax / 127), with amax the block's largest |x| in float32, the
  division an IEEE float32 division and the conversion to fp16 round-to-nearest-even;
- code q = round-half-even(x / s), dividing by the stored fp16 scale (as float32), and
  clamped to [-127, 127]; a block with s = 0 gets all codes 0.
Decoding is x_hat = q * s.
"""

import numpy as np

QBLOCK = 32


def q8_0_encode(k):
    """k: fp16 array [..., d] with d % 32 == 0.

    Returns (codes int8 [..., d], scales fp16 [..., d/32]).
    """
    k = np.asarray(k)
    if k.dtype != np.float16:
        raise TypeError("keys must be fp16")
    d = k.shape[-1]
    if d % QBLOCK:
        raise ValueError("head_dim must be a multiple of 32")
    x = k.astype(np.float32).reshape(k.shape[:-1] + (d // QBLOCK, QBLOCK))
    amax = np.max(np.abs(x), axis=-1)                      # float32, exact
    s16 = (amax / np.float32(127.0)).astype(np.float16)    # fp32 divide, RNE to fp16
    s32 = s16.astype(np.float32)[..., None]
    safe = np.where(s32 == 0, np.float32(1.0), s32)
    q = np.rint(x / safe)                                   # fp32 divide, half-to-even
    q = np.where(s32 == 0, np.float32(0.0), q)
    q = np.clip(q, -127, 127).astype(np.int8)
    return q.reshape(k.shape), s16


def q8_0_decode(codes, scales) -> np.ndarray:
    """fp64 [..., d] reconstruction q * s."""
    codes = np.asarray(codes)
    d = codes.shape[-1]
    q = codes.astype(np.float64).reshape(codes.shape[:-1] + (d // QBLOCK, QBLOCK))
    s = np.asarray(scales).astype(np.float64)[..., None]
    return (q * s).reshape(codes.shape)
