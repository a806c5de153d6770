"""Hardware probes behind the roofline figures (not part of the estimator)."""
