"""CPU fp64 oracle of Fibonacci-offset dilated sparse attention.

TEST INFRASTRUCTURE ONLY: only tests/, __graft_entry__.smoke() and the cpu_baseline leg of
bench.py may import or run anything in this package. The HIP library and its Python binding
never import it, and the two share no code.

Parity status: every function in fib_oracle is pinned by tests/test_oracle_*.py against
values fixed independently of it: brute-force membership and brute-force masks (index_sets
cell by cell in both modes), closed forms, library special cases, hand-derived constants,
finite differences and torch autograd.
"""
from .fib_oracle import *  # noqa: F401,F403
from .fib_oracle import __all__  # noqa: F401
