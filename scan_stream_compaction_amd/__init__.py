"""MI355X-native single-pass scan, stream compaction and stable partition."""
