"""CPU oracle for the Deja Vu sparse decode step: test infrastructure only.

Only tests/, __graft_entry__.smoke() and bench.py's CPU-baseline leg may import it.
"""
