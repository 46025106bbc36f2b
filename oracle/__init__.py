"""CPU oracle (test infrastructure only; see lemo_oracle's header)."""
