"""fp64 CPU oracle of the hybrid attention.  Test infrastructure only: the
product path never imports it."""
from . import rola  # noqa: F401
