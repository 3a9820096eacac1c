"""libpisa: PISA's pyramid Top-K block selector for MI355X (gfx950).

The compute path is the C-ABI shared library ``libpisa.so`` (HIP kernels, see
``include/pisa.h``); ``block_selection_pyramid_amd.pisa`` is its thin Python binding
(torch supplies device memory and the stream).  ``synth`` builds seeded synthetic
inputs.  Importing this package does not import torch.
"""

__all__ = ["pisa", "synth"]
