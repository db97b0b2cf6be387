"""MI355X-native selective state-space (S6) forward pass: HIP kernels for gfx950 behind a C ABI."""
