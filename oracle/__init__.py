"""Plain fp64 CPU oracle for one decode step of certified sparse attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or link
this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP path;
the two agree only through the written rules stated in the docstrings below.

Sources, cited by page and section (no other citation style is used here):

* [S]  "Certified Sparse Attention via Perturbed Retrieval", structured summary of
  the paper: sections Theoretical Foundation; Methodology > Problem Setup;
  Methodology > Algorithm Components items 1-4; Theorems 1-4.
* [A]  "Certified Sparse Attention via Perturbed Retrieval", the authors'
  abstract (GQA-shared 4-bit scan, fresh perturbations per step).

Where the pages leave a step open, the reading taken is stated where it is used.

Pinned against something other than itself in ``tests/test_oracle_*.py``:
dense attention (library softmax), pack (exact rational residual norms), score
bounds (brute force over every key), hash (published SplitMix64 outputs, KS test),
inclusion probability, HT unbiasedness and variance, nesting, the small-tau
limit, the error identity behind beta, the KL roots (library root finder),
certificate coverage per tail and per measure at a loose level, each measure's
beta against the worst case its event allows (brute force), the per-level budget
against the tails each measure's bound uses (union bound), Pinelis's tail at the
relaxed root, closed forms when no light key is sampled, the empirical
failure rate per measure at delta (Theorem 4) with planted mistakes that fail, and
the 8-bit tier (code rounding and the residual norm by exact rationals, bound
validity and the absence of false negatives by brute force over every key, the
relations between the sample, the exact reads and the 8-bit reads).
Parity unpinned against the pages: the specific constants of the certificate
completion (the per-level tail split, the centre, the G and Q tails) and the
hash -- the pages print no numbers for them; they are pinned by the rigour checks
above and by agreement with the HIP path.
"""

from .canon import LN2, RSQRT_D, PADF, csum128, logtau, first_level  # noqa: F401
from .dense import dense_attention, dense_attention_heads, exact_scores  # noqa: F401
from .pack import pack_kv_4bit  # noqa: F401
from .bounds import refine_bounds8, scan_bounds  # noqa: F401
from .perturb import splitmix64_mix, hash_prefix, perturbations  # noqa: F401
from .certify import kl, kl_upper_root, kl_lower_root, level_certificate, level_certificates, tails_per_level  # noqa: F401
from .decode import certified_decode, certified_decode_layer, level_sums, scan_stage, sample_stage  # noqa: F401
