"""sp24: 2:4 structured-sparse prune/compress and sparse GEMM for AMD MI355X (gfx950)."""
