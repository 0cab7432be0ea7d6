"""CPU oracle of the DFlash drafter pass (fp64, NumPy).  TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may import this
package.  The HIP library and its Python binding never import it, and it imports nothing from them.
"""
from .dflash_ref import *  # noqa: F401,F403
from . import ddtree  # noqa: F401,E402
from . import sampling  # noqa: F401,E402
from . import tree_attention  # noqa: F401,E402
