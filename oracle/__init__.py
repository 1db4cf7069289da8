"""CPU oracle for one denoise step of a block-autoregressive, uniform-state discrete-diffusion LM.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import or run anything in this package.  It shares no code with the HIP
path (no kernels, headers, helpers, tables or pre/post-processing) and imports nothing from it;
tests hand both sides the same seeded inputs.

Everything here is plain and slow on purpose: float64 NumPy arithmetic with library matmuls as
the only primitives, no blocking, fusion or reordering.  Where a floating-point value decides an
integer (the Gumbel-max token, the commit ranking, the re-noise threshold) the decision is taken
in float32, the precision the GPU kernels take it in.

Sources (the pages describing the method; cited by tag throughout):

* [GUIDE]  "DiffusionGemma Guia do Desenvolvedor para Decodificação Paralela a 1000+ Tokens/s"
           (dev.infolabhq.com) — sections "Arquitetura em Detalhes" (uniform-state diffusion,
           block-autoregressive diffusion) and "Demonstração: Resolvendo Sudoku…" (bidirectional
           context, re-noising).
* [NEWS]   "Google's DiffusionGemma Atinge 1.000 Tokens por Segundo" (aiexpert.news) — second
           paragraph (causal prefill into the KV cache, bidirectional 256-token canvas, commits
           of high-confidence tokens used as anchors, re-noising, block commit to the KV cache).
* [RANK]   "DiffusionGemma: geração de texto até 4x mais rápida…" (pulsar-ranking.com) —
           "Pontos-chave" (every token of the block attends to every other; iterative
           consolidation of correct tokens).
* [DOCS]   Google's DiffusionGemma documentation page (ai.google.dev/gemma/docs/diffusiongemma)
           — feature list (MoE backbone, autoregressive encoder + bidirectional canvas
           denoising) and the table "Configuração de exibição recomendada" (max 48 steps,
           linear temperature 0.8 → 0.4, adaptive early stop, token selection).

Parity status per function is listed in the module docstrings.  The full denoise step as a whole
has no worked numbers on the pages ("parity unpinned" for the composed step); each of its parts
is pinned by the tests in ``tests/test_oracle_*.py`` to closed forms, brute force, library
routines, published known-answer vectors and invariants.
"""

from . import philox, model, sampler, generate  # noqa: F401
