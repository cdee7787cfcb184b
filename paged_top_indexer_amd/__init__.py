"""MI355X-native QSA sparse-attention decode: paged top-512 block selection
and sparse attention over the selected tokens, as hand-written HIP kernels
for gfx950 behind a small C ABI (``include/qsa.h``)."""
