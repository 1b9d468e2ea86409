"""MI355X-native memory-efficient linear GRPO loss.

Thin ctypes binding over libgrpo.so (the C ABI in include/grpo.h).  Functions with
the C names (``grpo_advantages``, ``grpo_loss_fwd``, ``grpo_loss_bwd``,
``grpo_workspace_bytes``) only marshal tensors into pointers and sizes; every step
of the computation runs in the library's HIP kernels.  PyTorch provides device
memory and the current stream.  ``grpo_loss`` wraps the three calls in an
autograd function.

Importing this package loads the library and fails loudly if it is not built
(``python grpo_loss_amd/build.py``); there is no fallback.
"""

from ._binding import (  # noqa: F401
    GRPOError,
    GRPOOptions,
    KernelTrace,
    TRACE_KERNELS,
    grpo_advantages,
    grpo_grad_restore,
    grpo_loss,
    grpo_loss_bwd,
    grpo_loss_fwd,
    grpo_loss_fwd_bwd,
    grpo_loss_fwd_noalloc,
    grpo_quantize_e4m3,
    grpo_restore_workspace_bytes,
    grpo_scale_grad,
    grpo_workspace_bytes,
    library_path,
    load_library,
    offload_stream,
    options,
)
