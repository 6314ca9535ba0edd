"""tgemm: fp16 dense tiled matrix product for MI355X (gfx950)."""
