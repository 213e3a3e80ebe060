"""Feature-axis projected softmax attention (SPA / PDA style) for MI355X (gfx950)."""
