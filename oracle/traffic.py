"""Algorithmic HBM bytes and FLOPs of one MSA layer step.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: "vLLM 為 MiniMax-M3.1-Flash 提供 Day-0 支援" (English post),
section "MSA primer": every decode step reads the index key of each context
token (128 B per token per layer in FP8) -- one eighth of what dense attention
reads for that token's K/V (1,024 B: 4 KV heads x 128 dims in FP8) -- plus the
K/V rows of just the 2,048 chosen keys; at long context that is about 12.5%
of the dense traffic.  Section "What is new in the MiniMax-M3.1
architecture": NVFP4 needs 34,560 bytes per token where FP8 needs 61,440,
i.e. 4.5 bits per element instead of 8.

"Algorithmic" bytes are what the method itself must move: each index key
once, each selected K/V row once per (token, group) that selects it (distinct
rows only where stated), queries, outputs and the small metadata.  Repeat
reads and the per-key scores (never materialised) are not counted.
"""
KV_HEADS = 4
HEAD_DIM = 128

# bytes per element of one 128-dim row; NVFP4 = 64 B of codes + 8 B of scales
ROW_BYTES = {"f32": 4 * HEAD_DIM, "fp8": HEAD_DIM, "nvfp4": HEAD_DIM // 2 + HEAD_DIM // 16}


def index_key_bytes_per_token(dtype):
    """Index-key bytes per token per layer (one shared 128-dim head)."""
    return ROW_BYTES[dtype]


def kv_bytes_per_token(dtype, heads=KV_HEADS):
    """K plus V bytes per token per layer for ``heads`` KV heads."""
    return 2 * heads * ROW_BYTES[dtype]


def dense_decode_bytes(L, dtype):
    """K/V bytes dense attention reads for one decode step of length L."""
    return L * kv_bytes_per_token(dtype)


def sparse_decode_bytes(L, dtype, idx_dtype=None, max_keys=2048):
    """Index-key scan of the whole context plus full K/V of the selected keys."""
    idx_dtype = idx_dtype or dtype
    return L * index_key_bytes_per_token(idx_dtype) + min(L, max_keys) * kv_bytes_per_token(dtype)


def sparse_to_dense_ratio(L, dtype, idx_dtype=None):
    return sparse_decode_bytes(L, dtype, idx_dtype) / dense_decode_bytes(L, dtype)


def indexer_bytes(seq_lens, T, idx_dtype, q_dtype, groups, max_blocks):
    """Index keys of every sequence once + index queries + block scores written."""
    qb = 4 if q_dtype == "f32" else 1
    B = len(seq_lens)
    return (sum(int(L) for L in seq_lens) * ROW_BYTES[idx_dtype]
            + B * T * groups * HEAD_DIM * qb
            + B * T * groups * max_blocks * 4
            + B * max_blocks * 4 + B * 4)


def topk_bytes(B, T, groups, max_blocks, k=16):
    return B * T * groups * max_blocks * 4 + B * T * groups * k * 4


def attention_bytes(keys_per_row, kv_dtype, q_dtype, B, T, heads, with_lse=False):
    """K+V rows for the given number of attended keys (summed over rows of one
    KV head), query read and fp32 output written."""
    qb = 4 if q_dtype == "f32" else 1
    return (2 * int(keys_per_row) * ROW_BYTES[kv_dtype]
            + B * T * heads * HEAD_DIM * qb
            + B * T * heads * HEAD_DIM * 4
            + (B * T * heads * 4 if with_lse else 0))


def indexer_flops(total_query_key_pairs, groups):
    """2 * 128 flops per (query token, group, visible key)."""
    return 2 * HEAD_DIM * groups * int(total_query_key_pairs)


def attention_flops(total_head_key_pairs):
    """QK^T and PV: 4 * 128 flops per (query head, attended key)."""
    return 4 * HEAD_DIM * int(total_head_key_pairs)
