"""BitLinear forward on MI355X (gfx950): int8 x ternary, HIP kernels behind a
C-ABI library (``libug.so``).  The Python layer only marshals arguments."""
