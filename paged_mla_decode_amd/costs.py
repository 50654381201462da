"""Work and traffic counts for decode attention: the cost model behind the
benchmark's roofline (algorithmic bytes and flops per launch).

Plain host arithmetic, no device code. Units: bytes, multiply-accumulates
(MAC), flops (2 per MAC), seconds. "KB" here is 1024 bytes, "GB" 1e9 bytes,
"TB/s" 1e12 bytes/s, as in the worked examples these functions reproduce
(tests/golden/cost_examples.json).
"""
from __future__ import annotations

# DeepSeek-V2/V3 MLA shape.
KV_LORA_RANK = 512
QK_ROPE_HEAD_DIM = 64
QK_NOPE_HEAD_DIM = 128


def absorb_macs_per_query(num_heads: int, qk_nope_head_dim: int, kv_lora_rank: int) -> int:
    """MACs to fold W_UK into one query token: every head maps its no-rope
    query (qk_nope_head_dim) to kv_lora_rank values (SGLang v0.3 MLA page,
    exercise 1). Independent of the history length."""
    return num_heads * qk_nope_head_dim * kv_lora_rank


def decompress_macs_per_query(history: int, kv_lora_rank: int, num_heads: int,
                              qk_nope_head_dim: int) -> int:
    """MACs to rebuild every past token's per-head keys from its latent, the
    non-absorbed path (same exercise): history x kv_lora_rank x heads x dim."""
    return history * kv_lora_rank * num_heads * qk_nope_head_dim


def kv_bytes_per_token_layer(kv_heads: int, head_dim: int, elem_bytes: int,
                             tensors: int = 2) -> int:
    """Cache bytes one token adds to one layer: K and V (tensors=2) of every
    KV head (attention-backends page, what attention reads). For MLA the cache
    is one shared latent+rope row: kv_heads=1, head_dim=576, tensors=1."""
    return kv_heads * head_dim * tensors * elem_bytes


def mla_bytes_per_token(elem_bytes: int = 2, kv_lora_rank: int = KV_LORA_RANK,
                        rope_dim: int = QK_ROPE_HEAD_DIM) -> int:
    """One MLA cache row: the latent and the rope part, shared by all heads."""
    return kv_bytes_per_token_layer(1, kv_lora_rank + rope_dim, elem_bytes, tensors=1)


def decode_step_cache_bytes(batch: int, context: int, bytes_per_token: int) -> int:
    """A decode step reads every running request's whole cache once."""
    return batch * context * bytes_per_token


def seconds_at(nbytes: float, bytes_per_s: float) -> float:
    return nbytes / bytes_per_s


def break_even_context(weight_bytes: float, batch: int, bytes_per_token: int) -> float:
    """Context length at which a decode step's cache reads equal the weight reads."""
    return weight_bytes / (batch * bytes_per_token)


def ridge_flop_per_byte(peak_flops: float, bytes_per_s: float) -> float:
    """Flops per byte at which a kernel moves from memory-bound to compute-bound."""
    return peak_flops / bytes_per_s


def decode_flop_per_byte(query_heads_per_kv_head: int, head_dim: int, elem_bytes: int) -> float:
    """Arithmetic intensity of single-query decode per key: a head_dim-wide dot
    for the score and a head_dim-wide scaled add for the value (4*head_dim
    flops per query head) against head_dim-wide K and V rows. Query heads that
    share a KV head (GQA; all heads in MLA) reuse the same bytes."""
    flops = query_heads_per_kv_head * 4 * head_dim
    return flops / (2 * head_dim * elem_bytes)


def three_kernel_score_bytes(seq_len: int, elem_bytes: int) -> int:
    """One head's n x n score (or probability) matrix when attention is
    materialised in HBM (attention-backends page, FlashAttention)."""
    return seq_len * seq_len * elem_bytes


def qkvo_bytes(seq_len: int, head_dim: int, elem_bytes: int) -> int:
    """One head's Q, K, V and output: the only traffic of a fused kernel."""
    return 4 * seq_len * head_dim * elem_bytes


def three_kernel_traffic(seq_len: int, head_dim: int, elem_bytes: int) -> int:
    """HBM bytes per head of the three-kernel form: S and P each written once
    and read once, plus Q, K, V and the output."""
    return 4 * three_kernel_score_bytes(seq_len, elem_bytes) + qkvo_bytes(seq_len, head_dim, elem_bytes)


# ---- the path's own algorithmic counts (what the benchmark divides by time) ----

def mla_decode_latent_bytes(kv_tokens: int, cache_elem_bytes: int) -> int:
    """Latent bytes a decode launch must read: each used cache row once."""
    return kv_tokens * mla_bytes_per_token(cache_elem_bytes)


def mla_decode_flops(kv_tokens: int, num_heads: int) -> int:
    """Dense MFMA work of a decode launch: per token and head, the 576-wide
    score and the 512-wide latent-as-value product."""
    return 2 * num_heads * (KV_LORA_RANK + QK_ROPE_HEAD_DIM + KV_LORA_RANK) * kv_tokens


def absorb_bytes(rows: int, num_heads: int, head_dim: int = QK_NOPE_HEAD_DIM,
                 kv_lora_rank: int = KV_LORA_RANK, elem_bytes: int = 2) -> int:
    """W_UK, the no-rope query and the absorbed query, each once."""
    return elem_bytes * (kv_lora_rank * num_heads * head_dim + rows * num_heads * head_dim
                         + rows * num_heads * kv_lora_rank)


def project_bytes(rows: int, num_heads: int, head_dim: int = QK_NOPE_HEAD_DIM,
                  kv_lora_rank: int = KV_LORA_RANK, elem_bytes: int = 2) -> int:
    """W_UV, the latent output and the projected output, each once."""
    return elem_bytes * (kv_lora_rank * num_heads * head_dim + rows * num_heads * kv_lora_rank
                         + rows * num_heads * head_dim)
