"""pytest plugin of the host-sanitizer run (tests/test_sanitizers.py): the
loaders take the sanitized builds named by GDR_SANITIZED_LIBRARY and
GDR_SANITIZED_ORACLE in place of the in-tree libraries."""
import os


def pytest_configure(config):
    import gated_delta_rule_73_amd as gdr
    import oracle

    gdr.library_path = os.environ["GDR_SANITIZED_LIBRARY"]
    oracle._LIB = os.environ["GDR_SANITIZED_ORACLE"]


def pytest_sessionfinish(session, exitstatus):
    """Name the libraries the run actually loaded (checked by the caller)."""
    import gated_delta_rule_73_amd as gdr
    import oracle

    names = [getattr(gdr._lib, "_name", None), getattr(oracle._lib, "_name", None)]
    print(f"\nsanitized libraries loaded: {names}")
