"""MI355X-native gated delta-rule (GDN) prefill and decode.

The compute path is the C-ABI library ``libgdn.so`` (hand-written HIP for
gfx950) declared in ``include/gdn.h``; :mod:`gated_delta_rule_cte_amd.gdn` is
the thin Python binding over it.  Importing this package loads nothing; the
binding loads the library on first use and raises if it is not built.
"""
__version__ = "0.1.0"
