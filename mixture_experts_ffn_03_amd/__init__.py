"""MI355X-native mixture-of-experts FFN forward (HIP kernels behind a C ABI)."""
