"""CPU oracle package — test infrastructure only (see ``rmsnorm_oracle``)."""
from .rmsnorm_oracle import (backward, dgamma_from_rows, forward, forward_normed_rounded, inverse_rms, quantize,
                             weight)

__all__ = ["forward", "backward", "inverse_rms", "weight", "dgamma_from_rows", "quantize", "forward_normed_rounded"]
