"""MI355X (gfx950) tiled online-softmax attention forward.

The compute path is a HIP library (``libattn.so``, C ABI declared in
``include/attn.h``); this package only marshals torch tensors into it."""
