"""CPU oracle for jagged GDPA (test infrastructure only; see gdpa_ref.py)."""
