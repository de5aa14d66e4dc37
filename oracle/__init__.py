"""CPU oracle for the cached-prefix flow-matching denoise loop (TEST INFRASTRUCTURE).

This package is the plain, slow, obviously-correct float64 NumPy statement of
what the GPU path computes.  It exists only to check that path: nothing in the
product imports it; only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may call it.  It shares no code with the
HIP library: its only common dependency is the seeded input generator module
``synth`` (random draws, no arithmetic of the method).

Modules
-------
``expert``  the action expert and its Euler loop (schedule, timestep embedding,
            modulation tables, adaptive RMSNorm, GQA attention over the cached
            prefix plus the chunk, GeGLU MLP, in/out projections, update).
``joint``   the same velocity recomputed from prefix tokens every step in one
            masked joint sequence (the "no cache" formulation the cache must
            reproduce).
``int4``    offline round-to-nearest group-128 int4 quantiser and its
            dequantiser.
``wam``     the joint video/action denoiser with classifier-free guidance.

Every function cites the passage of the pages it follows.  The pages (three
web pages about PhyAI / FlashRT-PAI) describe the loop in prose only and print
no equations for the expert, so most constants are readings; each reading is
named where it is used.  Pinning (tests marked ``not gpu``): every function here
is checked against closed forms, invariants, brute force or library routines.
No function of this package is "parity unpinned".
"""
from . import expert, int4, joint, wam  # noqa: F401
