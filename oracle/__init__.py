"""Float64 CPU oracle of the tensor-parallel sharded linear layer (test infrastructure only).

Only the test suite, the smoke check and the CPU baseline leg of the
benchmark import this package; the HIP library and its binding never do.
"""
from .tp_oracle import *  # noqa: F401,F403
from .tp_oracle import __all__  # noqa: F401
