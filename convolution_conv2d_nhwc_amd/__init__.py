"""MI355X-native fused NHWC conv2d (dense KxK, 1x1, depthwise 3x3; fp32, bf16,
int8) behind a C ABI, plus the 4-tile mosaic packer.

The compute path is the HIP library ``libconv_nhwc.so`` built from ``csrc/``;
this package only marshals torch tensors into it. Importing the package does
not load the library; the first call that needs it does, and raises if the
library has not been built.
"""
from .data import Layer, Workload, WORKLOADS, workload  # noqa: F401


def __getattr__(name):
    # Lazy access to the binding so that the seeded data module can be used
    # on a machine where the HIP library is not built.
    if name in ("Conv2d", "ConvError", "mosaic_pack", "library_path", "lib", "STATUS", "DTYPES", "ACTS",
                "conv_out_shape", "pack_bias_scale"):
        from . import _lib
        return getattr(_lib, name)
    raise AttributeError(name)
