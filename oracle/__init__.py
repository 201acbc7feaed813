"""fp64 CPU oracle for VSA (test infrastructure; never on the product path)."""
