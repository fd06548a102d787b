"""CPU oracle for ReTopK decode attention (test infrastructure only; see retopk_oracle)."""
