"""MI355X-native chunked Gated DeltaNet forward (HIP kernels for gfx950 behind a C ABI)."""
