"""MI355X-native exact tiled attention (placeholder until the binding lands)."""
