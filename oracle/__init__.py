"""CPU oracle of the query-aware sparse-page decode path (TEST INFRASTRUCTURE).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import this package.
The product path (the HIP library and its Python binding) never imports, calls or links it.
"""
from .kvsel_oracle import *  # noqa: F401,F403
from .kvsel_oracle import __all__  # noqa: F401
