"""fp64 CPU oracle of the blocked Shampoo step (test infrastructure only).

Only the test suite, the package's smoke check and the benchmark's CPU
baseline import this package; the product path never does.
"""
from .shampoo_oracle import *  # noqa: F401,F403
from .shampoo_oracle import __all__  # noqa: F401
from .tensor_oracle import *  # noqa: F401,F403,E402
from . import tensor_oracle as _t  # noqa: E402

__all__ = list(__all__) + list(_t.__all__)
