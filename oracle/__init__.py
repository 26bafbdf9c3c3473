"""CPU oracle for MX block quantization (test infrastructure only).

Only the test suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import anything from this package. The library in
``microscaling_block_quantized_amd`` never imports it, and it imports nothing
from the library.
"""
from .mx_oracle import *  # noqa: F401,F403
from .mx_oracle import __all__ as _base_all
from .mx_variants import *  # noqa: F401,F403
from .mx_variants import __all__ as _variant_all
from .nvfp4 import *  # noqa: F401,F403
from .nvfp4 import __all__ as _nv_all
from .nested import *  # noqa: F401,F403
from .nested import __all__ as _nested_all

__all__ = list(_base_all) + list(_variant_all) + list(_nv_all) + list(_nested_all)
