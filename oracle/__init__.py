"""CPU oracle for the VGG-T^3 test-time-training layer.

TEST INFRASTRUCTURE ONLY. This package is the plain, slow, obviously-correct
reference that the HIP path is checked against. Only the test suite, the smoke
check and the benchmark's CPU-baseline leg may import it; the product library
never calls it and has no fallback to it. It shares no code with the HIP path.

Every function works in float64 from the exact input values (bf16 and fp32
inputs widen exactly), except the ShortConv2D, whose result is fixed bit for
bit by an fp32 evaluation contract (see ``shortconv``).

Parity pins: every function here is pinned by a CPU test against something
other than itself (brute force, closed forms, finite differences, library
routines, invariants); none is "parity unpinned".
"""
from .ttt import (  # noqa: F401
    bf16_round, shortconv, shortconv_direct, split_theta, join_theta,
    swiglu_forward, head_grad, ttt_grad, ttt_apply, ttt_write, ttt_read, ttt_loss,
    newton_schulz, muon_apply, NS_COEFFS, ttt_write_offload,
)
