"""Seeded synthetic inputs for paged decode attention.

This package only builds inputs: random K/V/q values, context lengths, a
seeded physical placement of pages, the block tables or raw slot tables that
record that placement, the new rows of the step and their slots, and the
copy list of a copy-on-write step.  It contains none of the attention
arithmetic and imports nothing from the library or from the oracle, so both
can consume the same scenario.
"""
from .configs import (CONFIG_NAMES, Scenario, Spec, build, config_spec,
                      make_config, random_spec, K_CANARY, V_CANARY)

__all__ = ["CONFIG_NAMES", "Scenario", "Spec", "build", "config_spec",
           "make_config", "random_spec", "K_CANARY", "V_CANARY"]
