"""Muon optimizer step for MI355X (gfx950): momentum, Frobenius normalisation,
Newton-Schulz orthogonalisation and the scaled write-back, as hand-written HIP
kernels behind a C ABI (libmuon_mi355x.so).  The Python layer only marshals
arguments; see `binding`."""
