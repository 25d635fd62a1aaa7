"""CPU oracle (test infrastructure only; see ringag_oracle.py)."""
