"""MI355X (gfx950) hybrid SWA/GA attention of MiMo-V2-Flash.

The compute lives in the HIP library ``libmimo_attn.so`` (C ABI declared in
``include/mimo_attn.h``); ``global_attention_mimo_amd.binding`` is the thin
ctypes binding over it.  ``synth`` draws the seeded synthetic inputs.
"""
