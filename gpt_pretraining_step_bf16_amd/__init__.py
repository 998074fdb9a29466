"""MI355X-native (gfx950) pretraining step of the depth-parameterised GPT.

The compute path is the HIP shared library built from csrc/ (C ABI declared in
include/gpt.h); ``binding`` marshals torch device tensors into it. Importing
this package does not load the library; ``binding.lib()`` does, and raises if
it has not been built.
"""
