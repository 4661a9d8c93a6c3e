"""MI355X-native sparse MLA (DeepSeek-V4 style) attention backward."""
