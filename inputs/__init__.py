"""Seeded synthetic inputs shared by the tests, the smoke check and the
benchmark.  Not part of the shipped library: it draws random numbers in the
shapes and distributions of the workloads and holds no step of the method."""
