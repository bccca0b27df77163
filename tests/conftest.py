import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_terminal_summary(terminalreporter):
    """Largest GPU-vs-oracle deviations seen by the comparison rules in this session."""
    mod = sys.modules.get("tests.parity")
    if mod is None or not mod.STATS["idx_compared"]:
        return
    st = mod.STATS
    terminalreporter.write_line(
        "parity: norm rel %.3g, gamma rel %.3g (err/tol %.3g), score err/tol %.3g; in-band index "
        "mismatches %d of %d, sign mismatches %d of %d, vectors with recomputed signs %d"
        % (st["norm_rel"], st["gamma_rel"], st["gamma_ratio"], st["score_ratio"], st["idx_mismatch"],
           st["idx_compared"], st["sign_mismatch"], st["sign_compared"], st["vectors_recomputed"]))
