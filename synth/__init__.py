"""Seeded synthetic input generators (no verification arithmetic)."""
