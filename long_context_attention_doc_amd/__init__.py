"""AnchorAttention for AMD MI355X (gfx950): a C-ABI HIP library plus a thin binding.

The attention pattern is the one of "When Precision Meets Position: BFloat16
Breaks Down RoPE in Long-Context Training" (arXiv 2411.13476): packed
documents with position IDs reset per document, RoPE on q/k, a shared anchor
token that every query sees, and no attention across documents.
"""
from .accounting import flops_fwd_bwd, unmasked_pairs_closed_form  # noqa: F401

__all__ = ["api", "accounting", "flops_fwd_bwd", "unmasked_pairs_closed_form"]


def __getattr__(name):
    if name == "api":
        import importlib
        return importlib.import_module(__name__ + ".api")
    raise AttributeError(name)
