"""Plain-kernel probes of what this GPU's memory system and matrix/vector
units deliver (bench.py reports them beside its rooflines). Measurement, not
part of the operator: nothing in gated_delta_rule_50_amd loads them."""
