"""Oracle: KV-cache capacity and utilisation arithmetic.

TEST INFRASTRUCTURE ONLY (see the package docstring).  These closed forms pin
the workload shapes (bytes per token, blocks per request) against the values
the pages print.
"""

from .paged_attention import num_blocks


def kv_bytes(layers, kv_heads, head_dim, tokens, element_bytes, requests=1):
    """Bytes of K and V for ``requests`` requests of ``tokens`` tokens each.

    Each layer keeps a K tensor and a V tensor, each with head_dim elements
    per KV head and token, so M = 2 * L * H_kv * T * d * b (KC, section
    "从张量元素数推导容量" (capacity from element counts)).  Every size must be
    a positive int (bool is not accepted as one); anything else raises
    ValueError.
    """
    sizes = {"layers": layers, "kv_heads": kv_heads, "head_dim": head_dim, "tokens": tokens,
             "element_bytes": element_bytes, "requests": requests}
    for name, value in sizes.items():
        if type(value) is not int or value < 1:
            raise ValueError(f"{name} must be a positive integer, got {value!r}")
    one_tensor = layers * kv_heads * head_dim * tokens * element_bytes  # K alone (or V alone), one request
    return 2 * one_tensor * requests


def kv_bytes_per_token(layers, kv_heads, head_dim, element_bytes):
    """KV bytes one token adds across all layers (XQ, "实践步骤" step 1)."""
    return kv_bytes(layers, kv_heads, head_dim, 1, element_bytes)


def reserved_utilisation(lengths, max_len):
    """Share of a max-length reservation that holds tokens (HB, "为什么要分页")."""
    return sum(int(t) for t in lengths) / (len(lengths) * int(max_len))


def paged_utilisation(lengths, block_size):
    """Share of allocated slots that hold tokens when paging.

    Each request holds ceil(T/B) blocks of B slots (HB, section "为什么要分页"
    (why paging), the utilisation estimate).
    """
    used = sum(int(t) for t in lengths)
    allocated = sum(num_blocks(t, block_size) * int(block_size) for t in lengths)
    return used / allocated
