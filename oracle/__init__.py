"""CPU oracle of Block Transformer inference.  TEST INFRASTRUCTURE ONLY: the GPU
path never imports it; only tests/, the smoke check and bench.py's CPU-baseline
leg do."""
from .model import *  # noqa: F401,F403
from . import model  # noqa: F401
