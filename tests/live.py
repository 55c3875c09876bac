"""Progress lines that reach the real output while pytest captures a test's
output: the long whole-tensor references and the name of each GPU case are
printed as they happen, not only when a test fails (test infrastructure)."""
import sys

_CONFIG = None  # set by conftest.pytest_configure


def line(msg: str) -> None:
    cfg = _CONFIG
    if cfg is not None:
        capman = cfg.pluginmanager.getplugin("capturemanager")
        reporter = cfg.pluginmanager.getplugin("terminalreporter")
        if capman is not None and reporter is not None:
            with capman.global_and_fixture_disabled():
                reporter.write_line(msg)
                reporter.flush()
            return
    print(msg, file=sys.stderr, flush=True)
