"""fp64 CPU oracle for the attention forward path.

TEST INFRASTRUCTURE ONLY: imported by the test suite, `__graft_entry__.smoke()` and the
`cpu_baseline` leg of `bench.py`, never by the product path. Shares no code with it.
"""
