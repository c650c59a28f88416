"""Float64 CPU oracle for attention backward -- test infrastructure only.

Only the tests, the smoke check and the benchmark's CPU-baseline leg use this
package; the GPU library never imports it.
"""
from .attention import *  # noqa: F401,F403
from .attention import __all__  # noqa: F401
