"""MI355X (gfx950) tree-causal draft-head hot path.

The compute lives in the HIP library ``libjf.so`` behind the C ABI declared in
``include/jf.h``; ``tree_causal_draft_parent_amd.jf`` is the thin Python
binding (argument marshalling only).  ``synth`` holds the seeded synthetic
input generators.  Importing this package loads nothing; the library is loaded
on first use and a missing library is an error, never a fallback.
"""
__all__ = ["jf", "synth"]
