"""CPU oracle (test infrastructure only; see leyline_oracle's header)."""
