"""CPU oracle of the constant-shape transformer decode step -- TEST INFRASTRUCTURE ONLY.

Only tests/, the graft entry point's smoke check and bench.py's CPU-baseline leg may import this package. The
product path (the HIP library and its Python binding) never imports, calls or executes anything here, and this
package imports nothing from the product path.
"""
from .decoder import *  # noqa: F401,F403
from .decoder import set_threads, threads  # noqa: F401
