"""Seeded synthetic workloads for the selective scan.

This package holds the five workload definitions (shapes, dtypes and value
distributions) and the seeded generators that draw their inputs, plus the
error metric used to compare two outputs.  It contains none of the scan's
arithmetic and imports neither the oracle nor the HIP binding; both sides
consume the very arrays generated here.
"""
from .configs import CONFIGS, Config, by_name, get_config  # noqa: F401
from .gen import backward_inputs, conv_inputs, forward_inputs, ssd_inputs, step_inputs, step_initial, bf16_bits_to_f64  # noqa: F401
from .compare import max_rel_err, err_report  # noqa: F401
