"""MI355X-native fused low-rank MoE router (MoRE) with top-k and gates.

The compute path is the HIP library ``libmore_route.so`` (C ABI declared in
``include/more_route.h``); ``rank_router_top_amd.route`` marshals torch device
tensors into it.  Importing this package does not load the library; the first
call does, and raises if the library is missing.
"""
__all__ = ["configs", "inputs"]
