"""CPU oracle for the BATQuant W4A4 deployment path — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import anything from this package.  The product path (the C-ABI
library and its Python binding) never imports, calls or links it, and this
package never imports the product path: the two share no code.  The only thing
they share is the seeded input generator package ``workloads``, which holds none
of the method's arithmetic.

``oracle.batquant`` is the plain vectorised fp64 form (NumPy; library matmuls as
single steps); ``oracle.scalar`` is a pure-Python loop form of the same
definitions, used on tiny inputs to cross-check the vectorised one.

Parity status of each function is stated in its docstring.  Every function here is
pinned by ``tests/test_oracle.py`` except where its docstring says
"parity unpinned".
"""
from . import batquant, scalar  # noqa: F401
