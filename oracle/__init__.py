"""CPU oracle package — test infrastructure only (see ``rmsnorm_oracle``)."""
from .rmsnorm_oracle import backward, dgamma_from_rows, forward, inverse_rms, weight

__all__ = ["forward", "backward", "inverse_rms", "weight", "dgamma_from_rows"]
