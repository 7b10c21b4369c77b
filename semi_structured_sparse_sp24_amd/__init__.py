"""2:4 semi-structured sparse GEMM for AMD Instinct MI355X (gfx950)."""
