"""Column-wise vocabulary top-k for speculative drafters on MI355X (gfx950).

The compute path is the HIP library libtopk_cols.so (C ABI declared in
include/topk_cols.h); `drafter_vocab_top_amd.topk_cols` is its ctypes binding.
`drafter_vocab_top_amd.workloads` builds the seeded synthetic inputs.
Submodules load lazily so that importing the package needs no GPU.
"""
__all__ = ["topk_cols", "workloads"]
