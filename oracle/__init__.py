"""Float64 CPU oracle for attention backward and the lightning-indexer backward -- test
infrastructure only.

Only the tests, the smoke check and the benchmark's CPU-baseline leg use this
package; the GPU library never imports it.
"""
from .attention import *  # noqa: F401,F403
from .attention import __all__ as _attention_all
from .indexer import *  # noqa: F401,F403
from .indexer import __all__ as _indexer_all

__all__ = list(_attention_all) + list(_indexer_all)
