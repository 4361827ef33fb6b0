"""The oracle: a plain, slow, obviously correct CPU model of PagedAttention decode.

TEST INFRASTRUCTURE ONLY.  Only `tests/`, `__graft_entry__.smoke()` and the
`cpu_baseline` leg of `bench.py` may import anything from this package.  The
product path (`paged_kv_cache_12_amd`, `libpa.so`) never calls it, and shares
no code with it: the oracle re-derives the cache layout, the pool policy and
the attention arithmetic from their definitions.

Modules
  attention  fp64 NumPy attention over block tables, cache layout reader and
             writer, block copy, split-K combine identity.
  pool_model pure-Python block pool with refcounts, fork / append / free and
             copy-on-write, under one fixed allocation policy.
  kv_size    per-token KV-cache size closed form.
  prefix_cache  chain-hash and radix-tree prefix indexes over the pool model.

Every function is pinned by `-m "not gpu"` tests against something other than
itself (brute force, invariants, closed forms, values printed on the pages,
element-by-element placement through hand-worked offsets).  Of the block
copies, `copy_blocks` is pinned by whole-block equality of each listed pair
and unchanged other blocks, `swap_blocks` element by element through the
hand-worked offsets: the direction of each pair, both K and V, whole blocks,
untouched blocks, pairs applied in order.
"""
