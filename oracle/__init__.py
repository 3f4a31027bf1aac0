"""fp64 CPU oracle (test infrastructure only; see hs_oracle)."""
