"""MI355X-native DFlash block-diffusion drafter forward.

The computation lives in ``libdflash.so`` (HIP kernels for gfx950 behind the C
ABI of ``include/dflash.h``); this package only marshals arguments.  Importing
it does not load the library; the first ``Drafter`` does, and fails loudly if
the library was not built.
"""
from .abi import ContextGap, DFlashError  # noqa: F401

__all__ = ["Drafter", "Session", "committed_batch", "flush_batch", "propose_batch", "sample", "select", "verify",
           "verify_noalloc", "WidthPolicy", "ContextGap", "DFlashError"]


def __getattr__(name):
    if name in ("Drafter", "Session", "committed_batch", "flush_batch", "propose_batch", "sample", "select", "verify",
                "verify_noalloc", "WidthPolicy"):
        from . import drafter
        return getattr(drafter, name)
    raise AttributeError(name)
