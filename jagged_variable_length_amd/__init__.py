"""jagged_variable_length_amd: jagged attention on MI355X (gfx950)."""
