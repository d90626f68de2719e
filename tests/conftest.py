import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TESTS_DIR = os.path.join(ROOT, "tests")
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# Size of the GPU suite.  A run of the whole suite with -m gpu that selects fewer tests is
# an error: a renamed or unregistered test file must not let the GPU suite pass by
# running nothing.
GPU_TESTS_MIN = 200

_gpu = {"selected": 0, "passed": 0, "skipped": 0, "failed": 0}


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_collection_finish(session):
    _gpu["selected"] = sum(1 for it in session.items if it.get_closest_marker("gpu"))


def pytest_runtest_logreport(report):
    if "gpu" not in report.keywords:
        return
    if report.when == "call" and report.passed:
        _gpu["passed"] += 1
    elif report.skipped:
        _gpu["skipped"] += 1
    elif report.failed:
        _gpu["failed"] += 1


def _whole_suite(config):
    args = [a for a in config.args if not a.startswith("-")]
    return bool(args) and all(os.path.abspath(a.rstrip("/")) == TESTS_DIR for a in args) \
        and not config.getoption("keyword")


def pytest_sessionfinish(session, exitstatus):
    config = session.config
    if config.getoption("markexpr") != "gpu" or config.getoption("collectonly"):
        return
    line = (f"GPU tests: {_gpu['selected']} selected, {_gpu['passed']} passed, {_gpu['skipped']} skipped, "
            f"{_gpu['failed']} failed")
    reporter = config.pluginmanager.get_plugin("terminalreporter")
    if reporter is not None:
        reporter.write_line(line)
    if _whole_suite(config) and _gpu["selected"] < GPU_TESTS_MIN and session.exitstatus == 0:
        if reporter is not None:
            reporter.write_line(f"error: the GPU suite selected fewer than {GPU_TESTS_MIN} tests")
        session.exitstatus = 1
