"""Seeded synthetic input generators (no indexer arithmetic)."""
