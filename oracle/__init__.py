"""CPU oracle of the fused MoE layer forward (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports, links or calls anything in here, and this
package imports nothing from the product.
"""

from .moe_oracle import *  # noqa: F401,F403
