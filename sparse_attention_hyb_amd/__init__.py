"""MI355X-native hybrid compressed/sparse + sliding-window attention (binding added with the C ABI)."""
