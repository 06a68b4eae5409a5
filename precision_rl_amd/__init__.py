"""MI355X (gfx950) per-token NVFP4 W4A4 MoE expert path.

The product is the C-ABI library ``lib/libw4a4moe.so`` (declared in
``include/w4a4_moe.h``); ``precision_rl_amd.binding`` is its thin ctypes
binding (imported explicitly, it needs torch), ``precision_rl_amd.synth``
draws the seeded synthetic inputs and ``precision_rl_amd.build`` compiles the
library.
"""
