"""One tensor-parallel rank's share of a Megatron-style GPT layer on MI355X.

The compute lives in the HIP library ``libtplayer.so`` (see ``include/tp_layer.h``);
``megatron_tensor_layer_amd.tplayer`` is its thin Python binding and
``megatron_tensor_layer_amd.inputs`` draws the seeded synthetic inputs.
Nothing is loaded at import time, so CPU-only tools can import the inputs
module without a GPU or a built library.
"""
