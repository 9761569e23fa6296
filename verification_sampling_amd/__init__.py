"""libspecverify for MI355X: the verify-and-speculate step of speculative
(and speculative speculative) decoding, as hand-written HIP kernels behind a
C ABI.  The binding lives in ``specverify``; importing this package loads
nothing."""

__all__ = ["specverify"]
