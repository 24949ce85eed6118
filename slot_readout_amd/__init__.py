"""MI355X (gfx950) denoise step, entropy-bounded commit and structured slot read.

``slot_readout_amd.dg`` is the ctypes binding of the C-ABI library libdg.so
(the same call names as include/dg.h); ``slot_readout_amd.runtime`` moves
inputs into device memory and allocates outputs and workspaces with torch.
Importing this package does not load the library; the first call does, and
fails loudly if it has not been built.
"""
__all__ = ["dg", "runtime"]
