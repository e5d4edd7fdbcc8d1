"""Late-layer KV cache fill for AMD MI355X (gfx950).

The fill of "RidgeFill: Training-Free Late-Layer Cache Fill for Faster
Prefill": for every row outside the exact set and every late layer, predict
the layer's input with a per-layer map, apply the layer's RMSNorm and key /
value projections, rotate the keys and store bf16 K/V in the layer's cache.
The work runs in hand-written HIP kernels behind the C ABI of include/rf.h
(librf.so); ``late_layer_kv_amd.binding`` is its ctypes binding.
"""
