"""KV-cache cost formulas used by the closed-form tests.

TEST INFRASTRUCTURE ONLY (see the oracle package docstring).

[AA] "Attention-head anatomy: one cache, four wirings", section 2: a token costs
2 * layers * kv_heads * head_dim * bytes of cache (one K and one V vector per
KV head per layer).  [DC] "MLA deep compression", "Decoupled RoPE" section, and
[AA] section 4: MLA replaces the 2 * kv_heads * head_dim block with d_c + d_R values
per layer.
Pinned by the worked numbers the pages print (tests/golden/cache_sizes.json).
"""


def kv_bytes_per_token(layers, kv_heads, head_dim, bytes_per_elem):
    """Per-token cache bytes of an MHA/GQA/MQA model."""
    return 2 * layers * kv_heads * head_dim * bytes_per_elem


def kv_elems_per_token_layer(kv_heads, head_dim):
    """Cached elements per token per layer of an MHA/GQA/MQA layer."""
    return 2 * kv_heads * head_dim


def mla_elems_per_token_layer(d_c, d_r):
    """Cached elements per token per layer of MLA: the latent plus the RoPE key."""
    return d_c + d_r


def mla_bytes_per_token(layers, d_c, d_r, bytes_per_elem):
    """Per-token cache bytes of an MLA model."""
    return layers * mla_elems_per_token_layer(d_c, d_r) * bytes_per_elem


def equivalent_gqa_groups(d_c, d_r, head_dim):
    """Number of GQA KV groups whose cache equals one MLA row: (d_c + d_r) / (2 head_dim)."""
    return mla_elems_per_token_layer(d_c, d_r) / (2 * head_dim)
