"""CPU oracle (test infrastructure only; see bsga_oracle's header)."""
