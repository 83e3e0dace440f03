"""MI355X-native masked second-order Higher-order Linear Attention.

The computation lives in libhla.so (hand-written HIP kernels for gfx950,
C ABI in include/hla.h); this package is its thin Python binding:

* :func:`forward_chunked` -- chunk-parallel masked forward (``hla_forward_chunked``)
* :func:`forward_chunked_noalloc` -- the same without a workspace (``hla_forward_chunked_noalloc``)
* :func:`backward_chunked` -- gradients with respect to q, k, v (``hla_backward_chunked``)
* :func:`attention` -- the two as one differentiable ``torch.autograd`` op
* :func:`decode_step` -- one streaming token per state (``hla_decode_step``)
* :func:`state_compose` -- masked semidirect-product composition (``hla_state_compose``)
"""
from ._binding import (EXPORTED, LIB_PATH, HlaError, State, attention, backward_chunked,
                       backward_workspace_size, decode_step, forward_chunked, forward_chunked_noalloc,
                       give_ups, load,
                       state_compose, workspace_size)

__all__ = ["EXPORTED", "LIB_PATH", "HlaError", "State", "attention", "backward_chunked",
           "backward_workspace_size", "decode_step", "forward_chunked", "forward_chunked_noalloc",
           "give_ups", "load",
           "state_compose", "workspace_size"]
