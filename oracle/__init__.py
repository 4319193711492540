"""CPU oracle (test infrastructure only): see knapspec_oracle."""
