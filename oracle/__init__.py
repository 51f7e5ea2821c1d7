"""CPU oracle of the drafter block (test infrastructure; see oracle.c header)."""
