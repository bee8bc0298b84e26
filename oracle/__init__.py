"""CPU oracle for batch-1 GPT-2 decode -- TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import
this package.  The product library (transformer_decode_token_amd) never imports,
links or calls it.
"""
from .oracle import Oracle, OracleLib, load_lib  # noqa: F401
