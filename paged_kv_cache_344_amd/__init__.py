"""MI355X-native paged decode attention: a C-ABI library (``libpa.so``) with gfx950 HIP
kernels, and this thin ctypes binding.  Importing the package does not load the
library; the first call does, and fails loudly when it is missing."""
