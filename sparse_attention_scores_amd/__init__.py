"""MI355X (gfx950) DeepSeek Sparse Attention layer step.

The compute lives in libdsa.so (hand-written HIP kernels behind the C ABI in
include/dsa.h).  ``sparse_attention_scores_amd.binding`` is a thin ctypes
layer over it; ``sparse_attention_scores_amd.workloads`` builds seeded
synthetic inputs shaped like GLM-5.x DSA layers."""
