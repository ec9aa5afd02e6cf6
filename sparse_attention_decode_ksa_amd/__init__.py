"""Block top-k / vote-union sparse decode attention for MI355X (gfx950)."""
