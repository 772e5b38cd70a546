"""MI355X-native MoE routing and dispatch-layout planning.

The hot path -- routing (top-K ids and weights), the padded per-expert layout with stable
permutation maps, and the expert-parallel plan over virtual ranks -- runs in hand-written HIP
kernels for gfx950 behind the C ABI declared in include/mep.h (libmep.so).  This package holds
the ctypes binding (``_binding``), the in-tree build (``build``) and the seeded synthetic input
generators (``synth``).  Importing the package does not load the library; the first call does,
and it raises if the library was not built.
"""

__all__ = ["route", "build_layout", "plan", "mep_route_topk", "mep_build_layout", "mep_plan"]


def __getattr__(name):
    if name in __all__ or name in ("alloc_layout", "alloc_plan", "alloc_workspace",
                                   "layout_workspace_size", "plan_workspace_size", "route_params",
                                   "default_nvs", "dedup_capacity", "MepError", "lib",
                                   "status_string", "permuted_capacity", "LayoutTensors",
                                   "PlanTensors", "MEP_SOFTMAX", "MEP_SIGMOID", "MEP_F32", "MEP_BF16"):
        from . import _binding
        return getattr(_binding, name)
    raise AttributeError(name)
