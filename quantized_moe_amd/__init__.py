"""MI355X-native W4A16 mixture-of-experts layer (HIP for gfx950).

``quantized_moe_amd.chord`` binds the C ABI of ``libchord.so``
(``include/chord.h``); ``quantized_moe_amd.build`` compiles it in-tree.
"""

__all__ = ["chord", "build"]
