"""Float64 CPU oracle (test infrastructure only; see fibattn_oracle's header)."""
