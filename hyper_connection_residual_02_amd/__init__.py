"""libhc: hyper-connection residual mixing on MI355X (gfx950)."""
