"""CPU oracle: plain fp64 reference of the relative-position memory attention.

Test infrastructure only: imported by tests/, by __graft_entry__.smoke() and by
bench.py's CPU-baseline leg; never by the product path.
"""
