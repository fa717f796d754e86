import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: larger CPU case")
    # Build only what is missing: a library that is already there is used as is.
    lib = os.path.join(ROOT, "gqa_attention_sinks_attn_amd", "libsink_attn.so")
    if not os.path.exists(lib):
        from gqa_attention_sinks_attn_amd import build as _b
        _b.build()
    import oracle
    oracle.build(force=False)
