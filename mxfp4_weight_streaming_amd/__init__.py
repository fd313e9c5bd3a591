"""MI355X-native (gfx950) W4A8 mixture-of-experts decode layer.

* ``binding``  -- the C ABI of libmoe_decode.so (hand-written HIP kernels);
                  importing it fails if the library is not built.
* ``synth``    -- seeded synthetic inputs of the measured workloads.
* ``build``    -- the hipcc build step for the library.
"""
__all__ = ["binding", "synth", "build"]
