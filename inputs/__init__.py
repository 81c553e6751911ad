"""Seeded synthetic input generators, shared by the oracle side and the GPU side.

Holds the data recipe and the storage encoding only; none of the product's
arithmetic lives here.
"""
