"""CPU oracle (float64) for XAttention block-sparse chunked prefill.

Test infrastructure only: imported by tests/, the smoke check and the
benchmark's cpu_baseline leg; never by the product path.
"""
