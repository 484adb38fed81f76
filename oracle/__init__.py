"""CPU oracle of the MSA hot path. Test infrastructure only: see msa_oracle.py."""
