"""MI355X-native denoise step of a block-autoregressive, uniform-state discrete-diffusion LM.

The compute path is the HIP library ``libdg.so`` (sources in ``csrc/``, C ABI in
``include/dg.h``); ``dg`` is its ctypes binding and ``synth`` draws seeded synthetic inputs.
Importing the package loads nothing; ``block_discrete_diffusion_amd.dg`` loads the library and
raises if it is missing.
"""
__all__ = ["dg", "synth"]
