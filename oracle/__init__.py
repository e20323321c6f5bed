"""Oracle package (test infrastructure only; see kvq_oracle's header)."""
