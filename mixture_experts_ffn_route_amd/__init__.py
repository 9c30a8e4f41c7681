"""MI355X-native (gfx950) DeepSeek-style MoE feed-forward layer forward pass.

The compute path is the HIP library ``libmoe_mi355x.so`` (C ABI in
``include/moe.h``); ``binding`` is its thin Python binding.  ``config`` holds
the layer configuration and the named workloads, ``synth`` the seeded
synthetic inputs.  Importing the package does not load the library; import
``mixture_experts_ffn_route_amd.binding`` for that.
"""

from .config import MoEConfig, Workload, FULL_WORKLOADS, SMALL_WORKLOADS

__all__ = ["MoEConfig", "Workload", "FULL_WORKLOADS", "SMALL_WORKLOADS"]
