"""MI355X-native verifier acceptance step (placeholder, binding added with the library)."""
