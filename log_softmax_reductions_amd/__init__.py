"""MI355X-native max-shifted log-sum-exp engine (placeholder; binding follows)."""
