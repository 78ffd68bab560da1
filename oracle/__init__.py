"""CPU oracle for the tensor-parallel sharded linear path (test infrastructure only).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import this package.
"""
from .tp_linear import *  # noqa: F401,F403
from .tp_linear import __all__  # noqa: F401
