"""MoE re-routing (MoeReRoutingV2) for MI355X: hand-written HIP kernels behind a C ABI.

`moe_re_routing` is the Python entry point (`moe_re_routing_inverse` runs the
moves backwards). The in-tree HIP library is loaded
on first use, and a missing build raises an error: there is no CPU fallback.
"""

_API = ("moe_re_routing", "moe_re_routing_inverse", "workspace_size", "get_device_status", "MrrError")


def __getattr__(name):
    if name in _API:
        from . import api

        return getattr(api, name)
    raise AttributeError(name)
