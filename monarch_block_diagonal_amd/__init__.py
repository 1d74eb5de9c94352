"""Monarch block-diagonal multiply for MI355X (gfx950)."""
