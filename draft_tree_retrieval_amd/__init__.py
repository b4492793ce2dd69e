"""Token Recycling (TR) draft-tree hot path for AMD MI355X (gfx950).

The work runs in libtr.so (hand-written HIP kernels behind the C ABI of
include/tr.h); `draft_tree_retrieval_amd.tr` is its Python binding.
"""
from . import tr  # noqa: F401
