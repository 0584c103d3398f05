"""fp64 CPU oracle for the fused linear epilogue and the LayerNorm+GELU row kernel.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything here. The
product path (the HIP library and its Python binding) never imports this
package and has no CPU fallback.

The oracle shares no code with the HIP path: it is plain numpy (fp64), with a
library matmul for the contraction and scipy's erf for the Gaussian CDF.
"""

from .fusedops_oracle import *  # noqa: F401,F403
