"""CPU oracle for the QSA hot path: test infrastructure only (see qsa_oracle)."""
