"""MI355X-native (gfx950) decode-step attention layer.

The layer (RMSNorm, Q8_0 activation quantization, Q5_0/Q8_0 block GEMVs with
bias, RoPE, KV-cache append, split-K GQA flash-decode attention, O projection
and residual add) runs in hand-written HIP kernels behind the C ABI declared in
``include/ck.h`` (``libck.so``). ``ck`` is the thin ctypes binding of that ABI;
``synth`` draws the seeded synthetic inputs. Importing the package loads
nothing: the library is opened on first use and its absence is an error.
"""
