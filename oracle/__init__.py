"""CPU oracle for IVF-PQ search (test infrastructure only; see oracle.py)."""
