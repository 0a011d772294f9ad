"""MI355X-native compressed sparse attention (DeepSeek-V4 CSA / HCA) layer path.

The kernels live in libcsa.so (C ABI in include/csa.h, HIP sources in csrc/); `binding`
marshals torch tensors into it and `pipeline` chains one layer step.
"""
from . import binding  # noqa: F401
