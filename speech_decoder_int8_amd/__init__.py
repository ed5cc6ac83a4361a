"""MI355X-native (gfx950) ARK-ASR-3B int8 decoder step.

The compute path is the HIP library libark.so (C ABI in include/ark.h);
`speech_decoder_int8_amd.ark` is its ctypes binding.  Build the library with
`python -m speech_decoder_int8_amd.build`.
"""
