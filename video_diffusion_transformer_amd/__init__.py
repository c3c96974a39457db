"""MI355X (gfx950) dense and block-sparse attention over video tokens."""
