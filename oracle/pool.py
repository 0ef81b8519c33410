"""The shared compressed pool: value bit-plane layout, byte counts, whole-pool helpers.

PolyKV, Abstract: the compressed cache is produced a single time and every agent reads
that one pool. The pages fix no byte layout; the one used here:
- key codes int8 [L][H][T][d] and key scales fp16 [L][H][T][d/32];
- value codes as three bit-planes over groups of 32 tokens: uint32 words
  [L][H][ceil(T/32)][3][d]; bit j of word (g, p, i) is bit p of the code of token
  32*g + j at coordinate i; bits of tokens past T are 0;
- value norms fp16 [L][H][T].
"""

import numpy as np

from .q8_0 import q8_0_encode, q8_0_decode
from .turboquant import tq_mse_encode, tq_mse_decode

TOKEN_GROUP = 32
PLANES = 3

# The pages' memory figures (PolyKV, Abstract): 2.91x compression; 19.8 GB -> 0.45 GB
# for 15 agents sharing a 4K context on Llama-3-8B; a 97.7% reduction. The 19.8 GB
# itself follows from nothing on the pages, so it is unpinned here.
PAGES_MEMORY_FIGURES = {"ratio": 2.91, "agents": 15, "gb_before": 19.8,
                        "gb_after": 0.45, "reduction_pct": 97.7}


def pack_v_planes(codes) -> np.ndarray:
    """codes uint8 [..., T, d] (values 0..7) -> uint32 [..., ceil(T/32), 3, d]."""
    codes = np.asarray(codes)
    *lead, T, d = codes.shape
    G = (T + TOKEN_GROUP - 1) // TOKEN_GROUP
    padded = np.zeros(tuple(lead) + (G * TOKEN_GROUP, d), dtype=np.uint32)
    padded[..., :T, :] = codes
    grouped = padded.reshape(tuple(lead) + (G, TOKEN_GROUP, d))
    out = np.zeros(tuple(lead) + (G, PLANES, d), dtype=np.uint32)
    for p in range(PLANES):
        bitp = (grouped >> np.uint32(p)) & np.uint32(1)
        word = np.zeros(tuple(lead) + (G, d), dtype=np.uint32)
        for j in range(TOKEN_GROUP):
            word |= bitp[..., j, :] << np.uint32(j)
        out[..., p, :] = word
    return out


def unpack_v_planes(words, n_tokens: int) -> np.ndarray:
    """Inverse of pack_v_planes: uint32 [..., G, 3, d] -> uint8 [..., T, d]."""
    words = np.asarray(words, dtype=np.uint32)
    *lead, G, P, d = words.shape
    codes = np.zeros(tuple(lead) + (G, TOKEN_GROUP, d), dtype=np.uint8)
    for p in range(P):
        for j in range(TOKEN_GROUP):
            bit = (words[..., p, :] >> np.uint32(j)) & np.uint32(1)
            codes[..., j, :] |= (bit << np.uint32(p)).astype(np.uint8)
    return codes.reshape(tuple(lead) + (G * TOKEN_GROUP, d))[..., :n_tokens, :]


def analytic_pool_bytes(n_layers: int, n_heads: int, n_tokens: int, head_dim: int) -> int:
    """Payload bytes: 1 B per key code, 2 B per 32-key scale, 3 bits per value code,
    2 B per value norm."""
    per_token = head_dim + 2 * (head_dim // 32) + (3 * head_dim) // 8 + 2
    return n_layers * n_heads * n_tokens * per_token


def fp16_kv_bytes(n_layers: int, n_heads: int, n_tokens: int, head_dim: int) -> int:
    return 2 * 2 * n_layers * n_heads * n_tokens * head_dim


def compress_pool(k, v, boundaries) -> dict:
    """Write-once compression of fp16 K and V [L][H][T][d] into the pool's arrays."""
    k_codes, k_scales = q8_0_encode(k)
    v_codes, v_norms = tq_mse_encode(v, boundaries)
    return {"k_codes": k_codes, "k_scales": k_scales,
            "v_codes": v_codes, "v_planes": pack_v_planes(v_codes), "v_norms": v_norms}


def dequant_pool(pool: dict, centroids, n_tokens=None):
    """Per-token reconstruction (fp64) of every key and value in the pool."""
    k_hat = q8_0_decode(pool["k_codes"], pool["k_scales"])
    if "v_codes" in pool:
        codes = pool["v_codes"]
    else:
        codes = unpack_v_planes(pool["v_planes"], n_tokens)
    v_hat = tq_mse_decode(codes, pool["v_norms"], centroids)
    return k_hat, v_hat


def dequant_fp16(pool: dict, centroids, n_tokens=None):
    """The pool as fp16 K and V, the form an ordinary per-layer cache holds (PolyKV,
    Abstract: the shared pool is handed to every agent as its KV cache).

    Each element is the fp64 reconstruction of dequant_pool rounded once, to nearest
    even, to binary16 (numpy's float64 -> float16 conversion rounds the double directly).
    For keys the fp64 value code * s is exact, so this is the correctly rounded result.
    """
    k_hat, v_hat = dequant_pool(pool, centroids, n_tokens)
    return k_hat.astype(np.float16), v_hat.astype(np.float16)


def append_pool(pool: dict, k_chunk, v_chunk, token_begin: int, boundaries) -> dict:
    """Write-once compression of one prefill chunk into tokens [token_begin, token_begin + n)
    of an existing pool of capacity T (PolyKV, Abstract: the cache is compressed a single
    time; here each chunk of the shared context is compressed once, when it arrives).

    pool: arrays as compress_pool returns them, with "v_codes" [L][H][T][d]; k_chunk and
    v_chunk: fp16 [L][H][n][d]. Every step of both codecs is per token, so the chunk's
    codes, scales and norms are those of compress_pool on the chunk alone; the planes are
    re-packed from the updated codes. Returns a new dict.
    """
    n = k_chunk.shape[-2]
    T = pool["k_codes"].shape[-2]
    if token_begin < 0 or n < 1 or token_begin + n > T:
        raise ValueError("token range outside the pool")
    part = compress_pool(k_chunk, v_chunk, boundaries)
    out = {key: np.array(val, copy=True) for key, val in pool.items()}
    sl = slice(token_begin, token_begin + n)
    out["k_codes"][..., sl, :] = part["k_codes"]
    out["k_scales"][..., sl, :] = part["k_scales"]
    out["v_codes"][..., sl, :] = part["v_codes"]
    out["v_norms"][..., sl] = part["v_norms"]
    out["v_planes"] = pack_v_planes(out["v_codes"])
    return out
