"""MI355X (gfx950) factored dictionary projection: Z = X D_g, Y = Z C_l.

The compute lives in the HIP library ``libdictfs.so`` behind the C ABI of
``include/dictfs.h``; ``binding`` is its thin ctypes binding (argument
marshalling only).  ``synth`` draws seeded synthetic inputs and ``ledger``
holds the byte / multiply-add accounting.  Importing the package loads
nothing; ``binding.lib()`` loads the library and raises if it is missing.
"""
__all__ = ["binding", "synth", "ledger"]
