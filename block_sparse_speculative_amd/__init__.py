"""Block-sparse multi-draft verification attention for MI355X (gfx950)."""
