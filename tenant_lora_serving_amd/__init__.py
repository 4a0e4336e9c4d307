"""Routed multi-tenant LoRA delta for MI355X (gfx950).

The library is the C-ABI shared object built from csrc/ (liblora.so); the
Python binding in `lora` marshals torch tensors to it.  Importing the package
does not load the library; `lora.lib()` does, and fails loudly when it is
missing.
"""
