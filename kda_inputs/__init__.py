"""Seeded synthetic inputs for the KDA mixer and their placement in device
memory.  Used by the tests, the smoke check and the benchmark; not part of
the library (`hybrid_linear_attention_rule_amd`), and free of the method's
arithmetic: the generators only draw and round numbers."""
