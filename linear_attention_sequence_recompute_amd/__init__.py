"""MI355X (gfx950) gated delta rule: chunked forward pass and recurrent decode step.

The computation runs in the HIP kernels of ``libgdn.so`` behind a C ABI
(``include/gdn.h``); ``api`` marshals torch tensors to it. ``workloads`` draws
seeded synthetic inputs.
"""

__all__ = ["chunk_fwd", "recurrent_step", "workspace_bytes", "GdnError"]


def __getattr__(name):
    if name in __all__:
        from . import api
        return getattr(api, name)
    raise AttributeError(name)
