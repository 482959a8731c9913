"""MI355X (gfx950) tensor-parallel transformer-layer shard.

One tensor-parallel rank's share of a Megatron-LM transformer layer (pre-LN
attention + MLP), forward and backward, and the vocabulary-parallel output
embedding fused with cross-entropy, as hand-written HIP kernels behind the C
ABI in include/tp_layer.h (libtplayer.so). ``binding`` is the ctypes layer;
``step`` sequences one pass of the path; ``build`` compiles the library.
"""
__all__ = ["binding", "step", "build"]
