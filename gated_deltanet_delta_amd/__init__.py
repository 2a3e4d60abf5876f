"""Gated delta rule on AMD Instinct MI355X (gfx950): a C-ABI HIP library and its Python binding."""
