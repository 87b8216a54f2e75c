"""libkda: Kimi Delta Attention (KDA) chunkwise prefill and recurrent decode for MI355X (gfx950).

The operator is the delta-rule recurrence with a channel-wise, lower-bounded forget gate of
Kimi K3: Open Frontier Intelligence, §2.1.1, eqs. (1)-(5).  Every step runs in hand-written HIP
kernels behind the C ABI declared in include/kda.h; this package only loads that library and
marshals torch tensors (device memory, streams) into it.

Submodules:
- binding : ctypes loader of libkda.so and the tensor-level wrappers (chunk_fwd, recurrent_step)
- inputs  : seeded synthetic input generators (no operator arithmetic)
- build   : compiles libkda.so for gfx950 with hipcc
"""

__all__ = ["binding", "inputs", "build"]


def __getattr__(name):
    # Load submodules lazily so that importing the package never touches the GPU library.
    if name in ("binding", "inputs", "build"):
        import importlib
        return importlib.import_module("." + name, __name__)
    if name in ("chunk_fwd", "chunk_fwd_workspace_size", "chunk_fwd_cp", "recurrent_step",
                "recurrent_multi_fused"):
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
