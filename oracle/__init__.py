"""CPU oracle for the gated delta rule.  Test infrastructure only (see oracle.py)."""
