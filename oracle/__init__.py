"""CPU oracle for one denoising step of confidence-guided, sink-aware block-sparse attention.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, obviously-correct CPU statement of what the
GPU path computes.  Only the test suite, the package's ``smoke()`` check and the benchmark's
CPU-baseline leg may import it; the product path (the HIP library and its Python binding) never
imports, links or executes anything here, and this package imports nothing from the product path.

Precision: attention outputs and sink masses are computed in float64 from the exact (bf16- or
fp32-valued) inputs.  Block / chunk / token scores are float32 with a pinned summation tree (see
``fp32tree``): products rounded to float32 before adding, no fused multiply-add, adjacent pairs summed
level by level.  Prediction and selection are exact integer / comparison logic.

Sources (cited by page title and section):
  * "Focus-dLLM: Accelerating Long-Context Diffusion LLM Inference via Confidence-Guided Context
    Focusing" -- the authors' abstract (chatpaper.ai page) and the Elamur Research page's "Summary"
    and "Key points";
  * "Prefilling-dLLM: Predictive Prefilling for Long-Context Inference in Diffusion Language Models"
    -- the abstract (fugumt.com and aiqbench.com pages).
The pages give no formula, pseudo-code or worked example, so every numeric detail is a reading;
each function names the reading it takes.

Pin status (what each function is checked against in tests/test_oracle_*.py):
  predictor        -- hand-worked cases, brute force over k-subsets
  fp32 tree        -- exact integer case, printed-order counterexamples, rounding error bound
  pooling / scores -- integer-valued inputs (exact under any order), error bound vs float64
  selection        -- hand-worked case, brute force over subsets, invariants
  sinks            -- row masses sum to 1, planted sinks recovered, pure-Python brute force
  attention        -- closed form, constant-V / zero-K cases, torch SDPA in float64, brute force
  chunked          -- all chunks + all tokens reduces to dense attention; page-order invariance;
                      token ranking on a strict chunk subset: hand-worked case and integer brute force;
                      shared chunks: integer brute force
Every function above is pinned.  What no pin can settle is whether the authors' own code takes the
same readings: the pages print neither formulas nor code, so that stays an open question about the
readings (each one is listed with its alternatives), not a gap in the oracle's pins.
"""
