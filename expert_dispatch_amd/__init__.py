"""MI355X-native routed-expert MoE layer (one expert-parallel rank, one GPU).

The hot path runs in the HIP library ``libmoe.so`` behind a C ABI declared in
``include/moe.h``; ``expert_dispatch_amd.ops`` is its thin Python binding
(argument marshalling only). ``workloads`` draws the seeded synthetic inputs.
Importing this package loads nothing: the library is opened on first use.
"""
__all__ = ["ops", "workloads"]
