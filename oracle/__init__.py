"""CPU oracle of the LSA indexer: test infrastructure, never the product path."""
