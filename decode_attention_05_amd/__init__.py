"""LowRAM decode path on MI355X (gfx950): HIP kernels behind a C-ABI library."""
