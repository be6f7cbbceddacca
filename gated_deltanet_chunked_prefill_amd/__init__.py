"""MI355X-native Gated DeltaNet chunked-prefill operator (placeholder; the
binding is added with the C-ABI library)."""
