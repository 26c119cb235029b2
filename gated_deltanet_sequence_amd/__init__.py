"""MI355X (gfx950) chunked gated-delta-rule forward pass and decode step.

The compute path is the C ABI of ``libgdn.so`` (declared in ``include/gdn.h``,
hand-written HIP kernels under ``csrc/``); :mod:`.binding` marshals torch
tensors into it.  :mod:`.inputs` holds the seeded synthetic workloads.

The binding is imported lazily so that the input generator can be used on
machines without the library or a GPU.
"""

__all__ = ["gdn_chunk_fwd", "gdn_recurrent_step", "GDNError", "load_library", "version"]


def __getattr__(name):
    if name in __all__:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
