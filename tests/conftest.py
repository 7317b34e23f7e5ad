import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


def gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="session")
def oracle_lib():
    import oracle
    return oracle.load()


def pytest_terminal_summary(terminalreporter):
    """One line per parity check of the run (pytest keeps a passing test's
    output to itself, so the records would otherwise not reach the log)."""
    parity = sys.modules.get("parity") or sys.modules.get("tests.parity")
    recs = getattr(parity, "RECORDS", None)
    grads = getattr(parity, "GRAD_RECORDS", None)
    tr = terminalreporter
    if grads:
        tr.write_sep("-", f"backward parity: {len(grads)} gradients against the fp64 oracle")
        tr.write_line(f"{'check':58s} {'grad':4s} {'max|err|':>9s} {'max|grad|':>9s} {'ratio':>9s} {'rel L2':>9s}")
        for what, name, err, scale, rel2 in grads:
            ratio = f"{err / scale:9.2e}" if scale >= 1e-6 else "        -"  # a gradient that is exactly 0
            tr.write_line(f"{str(what)[:58]:58s} {name:4s} {err:9.2e} {scale:9.2e} {ratio} {rel2:9.2e}")
    if not recs:
        return
    tr.write_sep("-", f"parity: {len(recs)} checks against the fp64 oracle")
    tr.write_line(f"{'check':58s} {'dtype':5s} {'elements':>10s} {'max|dO|':>9s} {'>1e-2':>6s} "
                  f"{'err/bound':>9s} {'max|dLSE|':>9s}")
    for r in recs:
        wb = r.get("worst_err_over_bound")
        tr.write_line(f"{str(r.get('what'))[:58]:58s} {r.get('dtype', ''):5s} {r.get('elements', 0):10d} "
                      f"{r.get('max_dO', 0.0):9.2e} {r.get('n_over_1e2', 0):6d} "
                      f"{(f'{wb:9.3f}' if wb is not None else '        -')} {r.get('max_dLSE', 0.0):9.2e}")
