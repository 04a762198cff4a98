"""CPU oracle for sparse MLA attention (test infrastructure only; see sparse_mla_oracle)."""
