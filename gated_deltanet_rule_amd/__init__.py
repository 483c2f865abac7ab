"""MI355X-native gated delta rule (Gated DeltaNet) hot path: chunked prefill,
packed recurrent decode and the mixed decode-plus-prefill step, as hand-written HIP
kernels for gfx950 behind a C ABI (``include/gdn.h``)."""
