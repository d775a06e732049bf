"""CPU oracle (test infrastructure only): see lrmoe_oracle."""
