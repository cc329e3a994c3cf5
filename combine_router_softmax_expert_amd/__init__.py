"""MI355X-native MoE expert-parallel dispatch and combine.

The path (router softmax/top-k, count, prefix sums, stable pack with a
combine handle, all-to-all-v exchange, expert stub, reverse exchange, weighted
top-k reduction) runs in the HIP kernels of libmoe_ep.so; ``binding`` is its
ctypes front end and ``workloads`` the seeded synthetic inputs.  The binding
is imported on first use of its names, so the input generator stays usable on
machines without the library.
"""

_BINDING_NAMES = {
    "Context", "MoeHandle", "MoeMeta", "MoeError", "moe_route_topk", "moe_dispatch", "moe_expert_stub",
    "moe_combine", "moe_dispatch_direct", "moe_dispatch_noalloc", "moe_combine_direct", "moe_dispatch_allgather", "moe_dispatch_send", "moe_dispatch_recv",
    "moe_combine_send", "moe_combine_recv", "moe_timing_begin", "moe_timing_end", "run_path", "run_overlapped", "lib",
}


def __getattr__(name):
    if name in _BINDING_NAMES:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
