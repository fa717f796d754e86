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


def pytest_terminal_summary(terminalreporter):
    """Parity of the five workloads (whole tensors where compared whole), so
    that the figures appear in the run's output even under -q."""
    from tests._helpers import PARITY_RECORD
    rows = [r for r in PARITY_RECORD if r[0].split()[0] in ("c1", "c2", "c3", "c4", "c5")]
    if not rows:
        return
    terminalreporter.write_line("parity against the fp64 oracle (max-abs <= 1e-2, rel-L2 <= 5e-3):")
    for name, n, mx, rl in rows:
        terminalreporter.write_line(f"  {name}: {n} values, max_abs={mx:.3e}, rel_l2={rl:.3e}")
