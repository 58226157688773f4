"""CPU oracle (test infrastructure only; see ix_oracle's header)."""
