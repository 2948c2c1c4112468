"""Oracle: a plain, slow, fp64 CPU reference for the ReplaySSM decode path.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in this
package. The HIP library never does, and this package imports nothing from it:
the two share no kernels, headers, helpers, tables or constants. Inputs come
from the seeded generators in ``workloads`` (which hold none of the method's
arithmetic), or from the tests themselves.

Sources. The method is known only from five web pages (the paper and its code
are not available). Citations name the page and the section on it:

  P1  "NVIDIA réécrit le stockage d'état des modèles hybrides"
      (blog.thibaultmonteiro.fr, French)
  P2  "ReplaySSM : l'IA qui cesse de réécrire son passé"
      (irisproject.cloud, French)
  P3  "ReplaySSM: Rethinking State Storage for Faster Hybrid-Model Decoding"
      (aikraft.ru, Russian)
  P4  "NVIDIA i Princeton eliminują wąskie gardła dekodowania w hybrydowych
      modelach SSM" (ainews.tenesys.com, Polish)
  P5  "Modèles à espace d'états vs Transformers : guide pratique"
      (datadaily.news, French)

Modules:
  mamba2  eager recurrence (the reference result), its unrolled closed form and
          semiseparable matrix, the checkpoint + ring replay model, the
          dual-precision and bf16-only-checkpoint emulators, the bf16-stored
          eager state, the speculative-stream reference
  ring    integer model of the per-sequence ring pointers
  lowp    bf16 round-to-nearest-even used by the low-precision emulators
  gdn     gated-DeltaNet eager rule and its replay model
  kda     Kimi Delta Attention (per-channel gated delta rule) and its replay model

Every function is pinned by ``tests/test_oracle_*.py`` to closed forms, exact
rational or 50-digit arithmetic, textbook special cases and invariants; none is
"parity unpinned".
"""
from . import lowp, ring, mamba2, gdn, kda  # noqa: F401
