"""Seeded synthetic inputs (the stand-in for the target model)."""
