"""lrsort: a stable LSD radix sort for AMD MI355X (gfx950)."""
