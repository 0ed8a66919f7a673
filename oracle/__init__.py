"""Float64 CPU oracle of HLTA.

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py, never by the GPU library or its binding.
"""
