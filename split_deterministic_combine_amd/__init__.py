"""Deterministic row reductions on MI355X (binding placeholder)."""
