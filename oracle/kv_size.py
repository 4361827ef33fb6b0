"""Per-token KV-cache size (test infrastructure only).

The vLLM encyclopedia entry (tonho.wtf), section "o problema", works the
OPT-13B case as two vectors (K and V) times the hidden size 5120 times 40
layers times 2 bytes in FP16.  "LLM : PagedAttention et RadixAttention
optimisent le cache KV", section "L'ampleur du cache KV fixe la concurrence des
services", names the factors as layers, KV heads, head dimension and bytes per
value.  Writing the hidden size as KV heads x head dim (40 x 128 for OPT-13B,
which has no grouped-query attention) gives one closed form.
"""


def kv_bytes_per_token(num_layers: int, num_kv_heads: int, head_dim: int,
                       elem_bytes: int) -> int:
    return 2 * num_layers * num_kv_heads * head_dim * elem_bytes


def kv_bytes(num_tokens: int, num_layers: int, num_kv_heads: int, head_dim: int,
             elem_bytes: int) -> int:
    return num_tokens * kv_bytes_per_token(num_layers, num_kv_heads, head_dim, elem_bytes)
