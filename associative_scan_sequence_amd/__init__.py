"""MI355X-native masked second-order Higher-order Linear Attention.

The computation lives in libhla.so (hand-written HIP kernels for gfx950,
C ABI in include/hla.h); this package is its thin Python binding:

* :func:`forward_chunked` -- chunk-parallel masked forward (``hla_forward_chunked``)
* :func:`forward_chunked_noalloc` -- the same without a workspace (``hla_forward_chunked_noalloc``)
* :func:`backward_chunked` -- gradients with respect to q, k, v (``hla_backward_chunked``)
* :func:`attention` -- the two as one differentiable ``torch.autograd`` op
* :func:`decode_step` -- one streaming token per state (``hla_decode_step``)
* :func:`decode_step_mq` -- the same with the key moment packed and shared by
  groups of query heads (``hla_decode_step_mq``; :func:`key_moment_pack` and
  :func:`key_moment_unpack` convert full and packed key moments)
* :func:`state_compose` -- masked semidirect-product composition (``hla_state_compose``)
* :func:`ahla_forward`, :func:`ahla_decode_step` -- the asymmetric variant (AHLA)
* :func:`third_forward`, :func:`third_decode_step` -- masked third-order HLA
"""
from ._binding import (EXPORTED, LIB_PATH, AhlaState, HlaError, MqState, State, ThirdState, ahla_decode_step,
                       ahla_forward, attention, backward_chunked, third_decode_step, third_forward,
                       backward_workspace_size, decode_step, decode_step_mq, forward_chunked,
                       forward_chunked_noalloc, give_ups, key_moment_pack, key_moment_unpack, load,
                       packed_size,
                       state_compose, workspace_size)

__all__ = ["EXPORTED", "LIB_PATH", "AhlaState", "HlaError", "MqState", "State", "ThirdState", "ahla_decode_step",
           "ahla_forward", "attention", "backward_chunked", "third_decode_step", "third_forward",
           "backward_workspace_size", "decode_step", "decode_step_mq", "forward_chunked",
           "forward_chunked_noalloc", "give_ups", "key_moment_pack", "key_moment_unpack", "load",
           "packed_size",
           "state_compose", "workspace_size"]
