import json
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; parity tests through the C ABI")


@pytest.fixture(autouse=True)
def _name_parity_records(request):
    from tests import _parity
    _parity.CURRENT_TEST[0] = request.node.nodeid
    yield


def _markdown(record):
    """One row per test function and compared quantity: over all its cases
    (parametrizations, heads), the comparison with the largest error / bound
    ratio, and the worst relative RMS error."""
    by = {}
    for test, rows in record.items():
        func = test.split("::", 1)[-1].split("[")[0]
        for name, err, rel, bound in rows:
            key = (func, name.split("[")[0].split(" ")[0])
            cnt, e, b, r = by.get(key, (0, -1.0, 1.0, 0.0))
            if bound > 0 and err / bound > e / b:
                e, b = err, bound
            by[key] = (cnt + 1, e, b, max(r, rel))
    lines = ["| test | quantity | comparisons | max abs error (worst case) | its bound | error / bound "
             "| worst relative RMS |", "|---|---|---|---|---|---|---|"]
    for (func, key), (cnt, e, b, r) in by.items():
        lines.append(f"| `{func}` | {key} | {cnt} | {max(e, 0.0):.3e} | {b:.3e} | {max(e, 0.0) / b:.3f} | {r:.2e} |")
    return "\n".join(lines) + "\n"


def pytest_sessionfinish(session, exitstatus):
    """With FA_PARITY_LOG set, write the achieved error of every comparison
    (max abs, relative RMS, bound) to that JSON file, and a Markdown table of
    the worst case per test and quantity next to it (same name, .md)."""
    path = os.environ.get("FA_PARITY_LOG")
    if not path:
        return
    from tests import _parity
    os.makedirs(os.path.dirname(os.path.abspath(path)), exist_ok=True)
    with open(path, "w") as f:
        json.dump(_parity.RECORD, f, indent=0)
    with open(os.path.splitext(path)[0] + ".md", "w") as f:
        f.write(_markdown(_parity.RECORD))
