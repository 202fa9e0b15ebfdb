"""MI355X (gfx950) implementation of the large-beam Gated DeltaNet decode step with shared-state
projection replay (OneLA).  The compute runs in the HIP library ``libonela.so`` behind a C ABI
(``include/onela.h``); ``linear_attention_beam_amd.onela`` is its thin ctypes binding and
``linear_attention_beam_amd.inputs`` the seeded synthetic workloads."""

__all__ = ["inputs", "onela"]
