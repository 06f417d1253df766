"""Plain CPU oracle of MoeReRoutingV2 (test infrastructure only)."""
