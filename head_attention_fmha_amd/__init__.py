"""MI355X (gfx950) fused multi-head attention: a C-ABI HIP library plus a thin ctypes binding."""
