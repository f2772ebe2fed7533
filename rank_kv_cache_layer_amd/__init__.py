"""MI355X-native per-hop KV-cache correction (KVCMAS hot path): HIP kernels behind a C ABI."""
