"""The oracle package exposes every function the parity tests, smoke() and
the benchmark call (a CPU check that no wrapper went missing)."""
import oracle


def test_module_functions_present():
    for name in ("softplus", "silu", "zoh", "selective_scan", "selective_scan_reverse",
                 "conv1d_silu", "conv1d_update", "state_update", "get", "build"):
        assert callable(getattr(oracle, name)), name
