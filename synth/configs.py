"""The five workload configurations, as plain data.

Shapes follow the attention layers of the models the Focus-dLLM pages evaluate (LLaDA-8B: 32 heads,
head_dim 128; Dream-7B: 28 query / 4 KV heads) at the 8K-32K contexts of Focus-dLLM's "Key points"
and Prefilling-dLLM's abstract, with 32-token decode blocks and a 256-token generation.  Values the
pages leave open (window, masked count, sink threshold ...) are fixed here and listed with their
reasons in the design notes.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace


@dataclass(frozen=True)
class Config:
    name: str
    seed: int
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ctx_len: int            # cached context tokens L
    dec_len: int            # decode-block tokens T
    kv_block: int           # tokens per KV block (selection unit)
    dtype: str              # "f32" or "bf16"
    top_k_pos: int          # predicted positions taken from the previous confidence
    window: int             # +/- widening around each predicted position
    top_k_blocks: int       # non-sink blocks kept per KV head
    sink_tau: float = 0.03  # mean softmax mass at or above which a cached token is a sink
    max_sinks: int = 64     # capacity of the sink-position list
    n_masked: int = 16
    conf_dist: str = "beta25"   # "uniform" or "beta25"
    sink_kind: str = "first4_x6"  # "shared_dir_x8" | "first4_x6" | "anchors"
    n_layers: int = 1
    dense_layers: int = 0   # leading layers that keep full attention
    source_layer: int = 0   # layer that detects sinks; deeper layers reuse them
    n_gen_blocks: int = 1
    steps_per_block: int = 1
    planted_blocks: int = 0
    planted_corr: float = 0.0
    paged: bool = False
    page_tokens: int = 0
    chunk_tokens: int = 0
    top_k_chunks: int = 0
    token_keep_frac: float = 0.0

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def n_blk(self) -> int:
        return -(-self.ctx_len // self.kv_block)

    @property
    def pages_per_seq(self) -> int:
        return self.ctx_len // self.page_tokens if self.paged else 0

    @property
    def n_pages(self) -> int:
        return self.batch * self.pages_per_seq

    @property
    def n_chunks(self) -> int:
        return self.ctx_len // self.chunk_tokens if self.chunk_tokens else 0

    @property
    def tokens_per_chunk_kept(self) -> int:
        """Non-anchor tokens kept inside each selected chunk: ceil(frac * chunk_tokens), at most all
        chunk_tokens - 1 non-anchor tokens."""
        return min(int(math.ceil(self.token_keep_frac * self.chunk_tokens)), self.chunk_tokens - 1)

    @property
    def max_sel_blocks(self) -> int:
        """Capacity for the selected-block list: every sink block plus the top-K."""
        return min(self.n_blk, self.max_sinks + self.top_k_blocks)

    def with_(self, **kw) -> "Config":
        return replace(self, **kw)


C0 = Config(name="tiny", seed=0, batch=1, n_q_heads=2, n_kv_heads=2, head_dim=64, ctx_len=512,
            dec_len=32, kv_block=32, dtype="f32", top_k_pos=4, window=2, top_k_blocks=4,
            conf_dist="uniform", sink_kind="shared_dir_x8")

C1 = Config(name="llada8b_8k", seed=1, batch=1, n_q_heads=32, n_kv_heads=32, head_dim=128,
            ctx_len=8192, dec_len=32, kv_block=64, dtype="bf16", top_k_pos=4, window=4,
            top_k_blocks=16)  # 12.5 % of 128 blocks

C2 = Config(name="dream7b_gqa_16k", seed=2, batch=1, n_q_heads=28, n_kv_heads=4, head_dim=128,
            ctx_len=16384, dec_len=32, kv_block=64, dtype="bf16", top_k_pos=4, window=4,
            top_k_blocks=32, planted_blocks=8, planted_corr=0.6)

C3 = Config(name="llada8b_32k_32layer", seed=3, batch=1, n_q_heads=32, n_kv_heads=32, head_dim=128,
            ctx_len=32768, dec_len=32, kv_block=64, dtype="bf16", top_k_pos=4, window=4,
            top_k_blocks=64, n_layers=32, dense_layers=2, source_layer=2, n_gen_blocks=8,
            steps_per_block=32, conf_dist="uniform")

C4 = Config(name="chunked_paged_32k_b4", seed=4, batch=4, n_q_heads=32, n_kv_heads=32, head_dim=128,
            ctx_len=32768, dec_len=32, kv_block=64, dtype="bf16", top_k_pos=4, window=4,
            top_k_blocks=0, sink_kind="anchors", paged=True, page_tokens=64, chunk_tokens=2048,
            top_k_chunks=4, token_keep_frac=0.25)

CONFIGS = {0: C0, 1: C1, 2: C2, 3: C3, 4: C4}


def get_config(i: int) -> Config:
    return CONFIGS[i]
