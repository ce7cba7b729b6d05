"""CPU oracle for chunked-prefill attention over a paged KV cache.

TEST INFRASTRUCTURE: only tests/, __graft_entry__.smoke() and the CPU-baseline
leg of bench.py may import anything from this package.
"""
