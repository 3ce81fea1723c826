"""CPU oracle for paged MLA decode: test infrastructure only (see mla_oracle)."""
