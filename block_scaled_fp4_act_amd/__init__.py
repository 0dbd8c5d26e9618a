"""Residue-compensated block-scaled FP4 linear for AMD Instinct MI355X (gfx950)."""
