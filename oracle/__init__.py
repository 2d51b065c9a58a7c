"""CPU oracle of the FastMKA layer forward -- test infrastructure only.

Imported only by the tests, the smoke check and the CPU-baseline leg of the
benchmark.  The HIP library never imports or calls it.
"""

from .mka_oracle import *  # noqa: F401,F403
