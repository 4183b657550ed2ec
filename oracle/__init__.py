"""CPU oracle for the single-GPU MoE layer forward (and backward of one workload).

TEST INFRASTRUCTURE ONLY. Nothing in the product path imports, calls, links or executes this
package; only the tests, the package's smoke check and the bench's CPU-baseline leg do. It shares
no code with the HIP library: no kernels, headers, helpers, tables or constant generators. Its only
common dependency with the GPU harness is the seeded input generator ``moe_inputs``, which holds
none of the method's arithmetic.

It is written to be read against the pages, not to be fast: plain NumPy in float64 (float32 only
where a fixed float32 order is itself the definition, see ``router_logits_fixed_order``), one
expert at a time, no blocking, fusion or reordering beyond what each definition states. The one
piece in C is the per-element E4M3 encoding and the per-block MX scale (``mx_codec.c``, plain loops
over elements and blocks, compiled with gcc without fast-math), so that the full-size weight
matrices can be quantised in seconds; ``formats.py`` states what it computes.

Sources. The method is the Mixture-of-Kittens MoE layer described on the page "Mixture-of-Kittens:
Cursor's Open-Source MoE Training Megakernel for NVL72" (sections TL;DR, the flowchart, Key claims)
and its companion articles. Those pages do not state the router formula, the top-k tie rule, the
SwiGLU definition or the MX element format; the workload definitions supply the first three
(softmax over router logits, top-k, renormalise; SwiGLU experts with W_gate, W_up, W_down) and name
E4M3 elements with one E8M0 scale per 32 elements, which the OCP Microscaling Formats (MX) v1.0 and
OCP 8-bit Floating Point (OFP8) v1.0 specifications define. Every further choice is marked
"Reading:" where it is made.

Parity status: every function is pinned by tests under tests/ against closed forms, brute force,
invariants or textbook special cases; none is "parity unpinned".
"""
from . import formats, moe  # noqa: F401
