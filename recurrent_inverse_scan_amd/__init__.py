"""MI355X (gfx950) Variational Linear Attention scan.

The compute lives in libvla.so (hand-written HIP kernels behind the C ABI of
include/vla.h); ``scan_forward`` and ``project_u`` marshal torch tensors into
it.  Importing the package does not load the library or touch the GPU.
"""
from .api import (fused_workspace_size, project_u, scan_backward, scan_forward, scan_forward_fused,  # noqa: F401
                  scan_step, timing_collect, timing_enable, workspace_size)
from .inputs import CONFIGS, ScanConfig, make_inputs  # noqa: F401
