"""MI355X-native exact tiled attention forward (gfx950 HIP kernel behind a C-ABI library)."""
