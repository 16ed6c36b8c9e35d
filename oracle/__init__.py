"""CPU oracle for the DiT denoise step -- test infrastructure only.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
import this package.  The product path (audio_latent_diffusion_amd) never
does, and shares no code with it.
"""
from .ald_oracle import *  # noqa: F401,F403
from . import ald_oracle  # noqa: F401
