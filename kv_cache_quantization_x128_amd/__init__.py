"""KVarN KV-cache tile codec for AMD Instinct MI355X (gfx950).

The codec runs as hand-written HIP kernels behind the C ABI declared in
``include/kvarn.h`` (``libkvarn.so``); :mod:`.kvarn` is the thin Python binding,
:mod:`.stream_cache` keeps an FP16 sink, the packed body and an FP16 trailing
window around it, and :mod:`.synth` generates seeded synthetic inputs.
"""
