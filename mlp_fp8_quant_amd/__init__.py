"""Static per-tensor FP8 (E4M3) W8A8 Linear stack for AMD MI355X (gfx950)."""
