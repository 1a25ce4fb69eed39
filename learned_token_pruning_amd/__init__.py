"""TokenGate pruned prefill for AMD Instinct MI355X (gfx950).

The compute lives in the HIP library ``libtokengate.so`` (C ABI, declared in
``include/tokengate.h``); :mod:`learned_token_pruning_amd.tokengate` is the
thin Python binding over it and :mod:`learned_token_pruning_amd.workloads`
draws the seeded synthetic inputs.  Importing this package loads nothing:
the binding loads the library when it is first imported and raises if the
library has not been built.
"""

__all__ = ["tokengate", "workloads"]
