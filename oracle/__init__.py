"""CPU oracle for the VideoMLA latent-KV chunk step (test infrastructure only;
see mla_oracle's header)."""
from .mla_oracle import *  # noqa: F401,F403
