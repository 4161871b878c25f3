"""MI355X-native MoE expert path: router -> dispatch -> grouped GEMM1 + SwiGLU ->
grouped GEMM2 -> weighted combine, forward and backward, as hand-written gfx950
HIP kernels behind a C ABI (``include/moe.h``).

Submodules:
  ``inputs``  seeded synthetic workloads (no method arithmetic)
  ``ops``     the Python binding of the C ABI (same names as the C entry points)
  ``layer``   ``MoEFunction``, a ``torch.autograd.Function`` whose forward calls
              ``moe_forward`` and whose backward calls ``moe_backward``

The binding is imported lazily so that ``inputs`` can be used without the HIP
library; any call into ``ops`` raises if the library is missing.
"""
