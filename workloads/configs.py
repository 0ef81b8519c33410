"""The five workload shapes.

The PolyKV abstract ("PolyKV: A Shared Asymmetrically-Compressed KV Cache Pool for
Multi-Agent LLM Inference", section "Abstract (arXiv)") evaluates SmolLM2-1.7B-Instruct
and Llama-3-8B-Instruct at contexts of 600 to 7,194 tokens (including a 4K context and
1,851 tokens) with up to 15 concurrent agents. The shapes below are those models' KV
shapes (layers, KV heads, head_dim, query heads per KV head) at those lengths.
"""

from dataclasses import dataclass


@dataclass(frozen=True)
class Config:
    index: int
    name: str
    n_layers: int
    n_kv_heads: int
    head_dim: int
    n_tokens: int
    n_agents: int
    gqa: int            # query heads per KV head
    decode_steps: int
    v_dist: str         # "normal" or "student_t4"

    @property
    def rows_per_tile(self) -> int:
        return self.n_agents * self.gqa

    @property
    def n_q_heads(self) -> int:
        return self.n_kv_heads * self.gqa

    @property
    def softmax_scale(self) -> float:
        return 1.0 / (self.head_dim ** 0.5)

    @property
    def kv_elems(self) -> int:
        return self.n_layers * self.n_kv_heads * self.n_tokens * self.head_dim


CONFIGS = (
    Config(0, "tiny", 1, 2, 128, 600, 1, 1, 1, "normal"),
    Config(1, "smollm2_1p7b_t600", 24, 32, 64, 600, 5, 1, 1, "normal"),
    Config(2, "llama3_8b_t1851", 32, 8, 128, 1851, 15, 4, 64, "normal"),
    Config(3, "llama3_8b_t4096", 32, 8, 128, 4096, 15, 4, 128, "normal"),
    Config(4, "llama3_8b_t7194_vt4", 32, 8, 128, 7194, 15, 4, 256, "student_t4"),
)


def config_by_name(name_or_index) -> Config:
    for c in CONFIGS:
        if str(c.index) == str(name_or_index) or c.name == name_or_index:
            return c
    raise KeyError(name_or_index)
