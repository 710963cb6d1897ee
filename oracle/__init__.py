"""fp64 CPU oracle for the ReHyAt hybrid attention forward.

TEST INFRASTRUCTURE ONLY: imported by tests/, the smoke check and the
benchmark's cpu_baseline leg, never by the library.  See oracle.py.
"""
