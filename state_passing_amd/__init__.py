"""MI355X-native chunkwise linear-recurrence layer with boundary state passing.

``state_passing_amd.linrec`` binds the HIP/gfx950 C-ABI library
(``include/linrec.h``); ``state_passing_amd.workloads`` draws the seeded
synthetic inputs.  Importing the package loads nothing; the first call into
``linrec`` loads ``liblinrec.so`` and fails loudly if it is missing.
"""
__all__ = ["linrec", "workloads"]
