"""What context parallelism moves per attention layer (forward), for sizing
the exchange around a rank share.

Zero to Frontier, "distributed/context-expert": section "What context
parallelism communicates" (a GPU's keys and values are 2 n d_kv numbers; the
ring and the all-gather both deliver the other n_cp - 1 of them) and section
"Ulysses, splitting by heads instead" (two all-to-alls of queries, keys,
values and output, each GPU keeping 1/n_cp of its share; Ulysses moves less
once the group is larger than 1 + h / n_kv).  Sizes in tokens and numbers,
bytes for elem_bytes per number (2 for 16-bit).
"""


def kv_block_bytes(n, d_kv, elem_bytes=2):
    """Keys plus values of n tokens with key/value width d_kv."""
    return 2 * n * d_kv * elem_bytes


def cp_comm_bytes(T, d, d_kv, n_cp, method, elem_bytes=2):
    """Bytes one GPU receives per layer: "ring" and "allgather" deliver the
    other n_cp - 1 key/value blocks; "ulysses" moves queries, keys, values and
    output of its n = T / n_cp tokens, all but its own 1/n_cp share."""
    if T % n_cp:
        raise ValueError("T must be a multiple of n_cp")
    n = T // n_cp
    if method in ("ring", "allgather"):
        return (n_cp - 1) * kv_block_bytes(n, d_kv, elem_bytes)
    if method == "ulysses":
        return 2 * n * (d + d_kv) * elem_bytes * (n_cp - 1) / n_cp
    raise ValueError(f"unknown method {method!r}")


def ulysses_breakeven(h, n_kv):
    """Group size above which Ulysses moves fewer bytes than the ring."""
    return 1 + h / n_kv


def overlap_min_tokens(F, B, h, n_kv):
    """Tokens per GPU above which a ring step's compute (4 n^2 d at F FLOP/s)
    hides its transfer (4 n d_kv bytes at B bytes/s): n >= (F / B)(n_kv / h)."""
    return F / B * n_kv / h
