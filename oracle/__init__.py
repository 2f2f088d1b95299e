"""CPU oracle of the CRISP sparse-prefill path (test infrastructure only)."""
