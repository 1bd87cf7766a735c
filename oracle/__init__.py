"""CPU oracle for the offloaded MoE layer -- TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously-correct NumPy (fp64 unless a step fixes another
precision).  It exists so the tests, the smoke check and the benchmark's CPU
baseline leg can compare the GPU library against an independent statement of
what the layer computes.  Nothing in the product path may import it; it shares
no code with the GPU library (only the seeded input generators in `moe_synth`
are common to both sides).

What it follows (page titles and sections of the FreeToken pages):
  * Router top-k, experts cached in a GPU LRU pool, misses streamed over PCIe,
    hybrid split of a step's misses, one global pool shared by all layers --
    devpik article "FreeToken: Run Frontier MoE Models on Your Own GPU, and the
    RAM It Takes", section "Why a Huge MoE Model Fits on One Consumer GPU";
    byteiota article "FreeToken: Run a 290B MoE Model on One Gaming GPU",
    sections "VRAM Is Not the Bottleneck You Think It Is" and "The
    Bandwidth-Adaptive Runtime".
  * Prefill: every MoE layer copies all of its experts per chunk, double
    buffered (layer N+1 copies while N computes) -- devpik article, section
    "Long Prompts Are the Bottleneck".
  * Number formats MXFP4 / NVFP4 / FP8 -- devpik article, "The Real Requirement
    Is System RAM" (NVFP4: an 8-bit scale per 16 weights); the bit-level
    encodings are those of the OCP Microscaling Formats (MX) v1.0 and OCP 8-bit
    Floating Point (OFP8) specifications.

Modules: formats (decode, bf16 rounding, MX activation quantiser), router
(fp64 logits, top-k, renormalised softmax), lru (step-set global LRU pool),
ffn (SwiGLU expert, combine), layer (a whole layer call and a workload run).

Parity status of every function is pinned by tests under tests/ (see each
module's docstring); the one deliberately unpinned claim is parity with the
FreeToken implementation itself, whose cache granularity, tie-breaks and split
rule are not published.
"""
