"""Plain, slow float64 CPU oracle for the branch-packed scoring pass.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or links
this package: only the tests, the smoke check and the benchmark's CPU-baseline
leg do.  It shares no code with the HIP path (``shared_prefix_branch_amd``) and
never reads a value the HIP path produced.

Sources are the three pages about the spinf-serve engine:
  [PyPI]    the project page "spinf-serve 0.1.1" on pypi.org;
  [man]     the man page "spinf-serve" on linuxcommandlibrary.com;
  [article] "Bulk classification and decision inference on one GPU" (the
            English original on aitujian.cn).
Each module cites the passages it follows.

Modules:
  numerics  -- exact bf16 / OCP e4m3fn decoding to float64
  tree      -- logical rows, option tries, tree parents and root paths
  attention -- branch attention: per-sequence form and dense-mask form
  scoring   -- logits, log-softmax, option log-probs, p, residual, floors, lift
  forward   -- the decoder stack around branch attention (rmsnorm, RoPE,
               projections, gated MLP) on synthetic weights
  decode    -- searched decoding of extraction slots (beam search)

Parity pins: every function here is pinned by a ``-m "not gpu"`` test against
something other than itself (the worked example on the article, closed forms,
library special cases, brute force on tiny inputs).  None is unpinned.
"""
from . import numerics, tree, attention, scoring, forward, decode  # noqa: F401
