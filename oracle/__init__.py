"""fp64 CPU oracle for the DiffusionGemma canvas denoise step.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything here.  The
HIP library never routes through this package, and this package imports
nothing from the HIP side: the two share no code.  The only module both use is
``synth_inputs`` (shapes and seeded prompt/logit inputs, no arithmetic of the
method).

Sources.  The pages are five web pages about Google's DiffusionGemma:
  [P1] "Diffusion Gemma - Google AI 教學課程" (ai-directories.com), Part 2 §2.1
       (diffusion principle table) and §2.2 (MoE / hardware table);
  [P3] "DiffusionGemma 是什麼？看懂 256-token Canvas 與本機 A/B Test"
       (alphalab.site), section "256-token Canvas 怎麼從雜訊變成文字？",
       steps ① to ④, and FAQ 2–3;
  [P4] MarkTechPost article in Arabic translation (k7ail.com), sections
       "how text diffusion works" and "architecture";
  [P5] Google launch blog in Vietnamese translation (aitoday.skyai.vn),
       sections "why diffusion for text" and "how text diffusion works".
Every function cites the passage it follows.  Points the pages leave open
take the plainest reading, stated in the docstring of the module that uses it.

Precision: everything is fp64.  Weights are held at their storage precision
(fp32, bf16, or e4m3 with a bf16 per-row scale) and used exactly as stored.

Parity status: every function here is pinned by tests under ``tests/`` that
check it against closed forms, brute force, library routines or invariants
(see each module's header).  The composition of the whole 30-layer forward at
full width has no independent pin beyond its component pins and invariants.
"""
