"""MI355X (gfx950) chunked gated-delta-rule forward pass and decode step.

The compute path is the C ABI of ``libgdn.so`` (declared in ``include/gdn.h``,
hand-written HIP kernels under ``csrc/``); :mod:`.binding` marshals torch
tensors into it.  :mod:`.inputs` holds the seeded synthetic workloads.

The binding is imported lazily so that the input generator can be used on
machines without the library or a GPU.
"""

__all__ = [
    "gdn_chunk_fwd", "gdn_chunk_fwd_split", "gdn_chunk_fwd_split_workspace", "gdn_chunk_fwd_split_noalloc",
    "gdn_scan_fwd", "gdn_scan_fwd_workspace", "gdn_scan_fwd_vecgate", "gdn_recurrent_fwd",
    "gdn_recurrent_fwd_vecgate",
    "gdn_chunk_fwd_vecgate", "gdn_chunk_fwd_vecgate_split", "gdn_chunk_fwd_vecgate_split_workspace",
    "gdn_chunk_fwd_vecgate_2pass", "gdn_chunk_fwd_vecgate_2pass_workspace",
    "gla_chunk_fwd", "gdn_recurrent_step", "gdn_recurrent_step_vecgate", "gla_recurrent_step",
    "GDNError", "load_library", "strerror", "version",
]


def __getattr__(name):
    if name in __all__:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
