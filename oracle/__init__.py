"""CPU oracle for the quantized linear layers (test infrastructure only).

Only the test suite, ``__graft_entry__.smoke()`` and ``bench.py``'s
``cpu_baseline`` leg import this package. It shares no code with the HIP
library and the library never imports it.
"""
from . import w8ref  # noqa: F401
