"""MI355X-native forward pass of one pre-LayerNorm ViT encoder block.

The computation runs in hand-written HIP kernels for gfx950 inside
``libvitblk.so`` (C ABI declared in ``include/vitblk.h``); this package is the
thin ctypes binding over it plus the seeded synthetic-input generator.
Importing the package does not load the library; the first call does, and it
raises if the library has not been built.
"""
