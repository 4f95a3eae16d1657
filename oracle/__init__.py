"""fp64 CPU oracle of the gated delta rule (test infrastructure only; the
product path never imports it)."""
