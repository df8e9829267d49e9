"""CPU oracle (test infrastructure only; see oscar_oracle's module docstring)."""
