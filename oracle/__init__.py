"""CPU oracle of the drafting path (test infrastructure; never on the product path)."""
