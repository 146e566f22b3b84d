"""MI355X-native real-time MoE expert load balancing (UltraEP-style hot path,
Waterfill shared-expert placement and LPLB replica split).

The compute path is the HIP library ``libuep.so`` (C-ABI, see ``include/uep.h``);
``moe_expert_load_amd.uep`` is its thin Python binding.  Importing this package
does not load the library; ``moe_expert_load_amd.uep`` does, and fails loudly
when it is missing.
"""

__version__ = "0.1.0"
