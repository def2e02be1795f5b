"""MI355X-native multi-scale deformable attention (MSDA) core: forward (plain,
fused front end, pruned), backward, the projections around it, and visit
orders for pixel-centre queries and for queries given by a point each.

The computation lives in ``libmsda.so`` (HIP, gfx950) behind the C ABI of
``include/msda.h``; ``binding`` marshals torch GPU tensors to it.
"""
from .binding import (MSDA_BF16, MSDA_F32, MsdaError, load_library, msda3d_backward,
                      msda3d_forward, msda3d_forward_fused, msda3d_forward_pruned,
                      msda_backward, msda_forward, msda_forward_fused, msda_forward_pruned,
                      msda_linear, msda_query_order, msda_query_order_points, status_string)

__all__ = ["msda_forward", "msda3d_forward", "msda_forward_pruned", "msda3d_forward_pruned",
           "msda_forward_fused", "msda3d_forward_fused", "msda_backward", "msda3d_backward",
           "msda_linear", "msda_query_order", "msda_query_order_points", "status_string", "load_library", "MsdaError", "MSDA_F32", "MSDA_BF16"]
