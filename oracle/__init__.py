"""fp64 CPU oracle of the WSVD low-rank decode step.

Test infrastructure: imported only by the tests, the package smoke check
and the benchmark's CPU-baseline leg.  Never part of the GPU path.
"""
from .wsvd_oracle import *  # noqa: F401,F403
from .wsvd_oracle import __all__ as _core_all
from .w8a8 import *  # noqa: F401,F403
from .w8a8 import __all__ as _w8a8_all
from .rope import *  # noqa: F401,F403
from .rope import __all__ as _rope_all
from .factorize import *  # noqa: F401,F403
from .factorize import __all__ as _fact_all
from .shared_svd import *  # noqa: F401,F403
from .shared_svd import __all__ as _shared_all

__all__ = list(_core_all) + list(_w8a8_all) + list(_rope_all) + list(_fact_all) + list(_shared_all)
