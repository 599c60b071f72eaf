"""CPU float64 oracle for block-sparse FlashAttention prefill.

TEST INFRASTRUCTURE: only ``tests/``, ``__graft_entry__.smoke()`` and the CPU
baseline leg of ``bench.py`` may import this package.  The HIP product path
never imports, links or executes it.  Every function cites the passage of
"Block Sparse Flash Attention" (paperpeel.com/paper/2512.07011) it follows.

Pins: each function here is checked by the ``tests/test_oracle_*.py`` files
against something other than itself (a library attention routine, closed
forms, a brute-force streaming loop, invariants and the pages' printed
figures); ``tests/test_oracle_mutants.py`` plants mistakes to show the pins
catch them.
"""

from .bsfa_oracle import *  # noqa: F401,F403
from .bsfa_oracle import __all__  # noqa: F401
