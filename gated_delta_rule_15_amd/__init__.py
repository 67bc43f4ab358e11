"""MI355X-native KDA recurrence library (HIP kernels behind a C ABI)."""
