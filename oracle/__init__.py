"""fp64 CPU oracle for span-routed mixed-resolution KV decode (SEKV form).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this package: only the test-suite, the smoke check and the bench's
CPU-baseline leg use it.  It shares no code, constants or helpers with the
HIP library; the two are compared on the same seeded inputs.

The submodule ``paris`` is the oracle of the token-retrieval router
(ParisKV page) and ``qevict`` that of the window-routed three-tier cache
(QEvict page); their readings and pinning status are in their own
docstrings.

Every function of the SEKV part follows a passage of the SEKV summary ("SEKV - KV Cache
Adattiva alla Risoluzione con Memoria Semantica Gerarchica", gist.science,
Italian and Korean editions), cited by section name in its docstring.

Pinning status (what fixes each function independently of itself):
  * segmentation       - pinned: hand-worked examples, brute-force rank
                          definition on tiny inputs, tie-heavy inputs.
  * summaries          - pinned: unit norm, equal-key and constant-weight
                          closed forms, scale invariance, ln|S| closed form.
  * truncated SVD      - pinned: matrices with a constructed SVD (known
                          singular values and vectors), Eckart-Young error,
                          orthonormal basis, exact reconstruction at full rank.
  * routing / top-k    - pinned: brute-force subset enumeration, tau = +-inf,
                          k_max = 0, basis-vector closed form for z.
  * attention          - pinned: torch's scaled_dot_product_attention (fp64,
                          GQA) when every token is an anchor or every span is
                          expanded at full rank; the equal-key closed form for
                          an unexpanded span; constant values; convex hull.
  * parity unpinned    - the readings themselves where the pages are silent:
                          raw-surprisal weights, the arithmetic mean as the
                          unexpanded value, the gate sigmoid(alpha<rho,s>-tau)
                          with a strict cut at 1/2, mean-of-group routing.
"""
from .sekv import *  # noqa: F401,F403
from . import paris  # noqa: F401  (ParisKV-style token retrieval, its own page)
from . import qevict  # noqa: F401  (QEvict-form window routing, its own page)
