"""CPU oracle of the mHC pre/post path (test infrastructure; see hc_oracle)."""
