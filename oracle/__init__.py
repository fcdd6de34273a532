"""CPU oracle for RaBiT-style 2-path residual binarization.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or link
anything under ``oracle/``; only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it. It shares no code with the HIP
path (``bit_residual_binarized_amd``) and imports nothing from it.

Parity pinning: every function here is checked by ``tests/test_oracle_*.py``
against something other than itself (closed forms, brute force with exact
rationals, independent library routines, invariants). See the module docstring
of ``oracle.rabit_oracle`` for which pin covers which function.
"""
from .rabit_oracle import *  # noqa: F401,F403
from .rabit_train import *  # noqa: F401,F403
from .rabit_init import *  # noqa: F401,F403
