"""fp64 CPU oracle of the KDA layer: test infrastructure, never on the product path."""
