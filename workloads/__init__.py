"""Seeded synthetic inputs (no Muon arithmetic)."""
