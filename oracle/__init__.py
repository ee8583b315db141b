"""CPU oracle of the MTGR HSTU layer: test infrastructure, never the product path."""
