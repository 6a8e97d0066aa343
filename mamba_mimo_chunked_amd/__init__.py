"""MI355X (gfx950) HIP implementation of the Mamba-3 MIMO backward first stage.

``mamba_mimo_bwd_fwd`` re-runs the chunked MIMO scan and returns the bf16
chunk entry states, the same-token qk_dot and the optional dmimo_o / dz /
dmimo_z gradients; ``mamba_mimo_fwd`` returns the layer output those
gradients belong to. The computation runs in the HIP library
``_build/libmimo_bwd_fwd.so`` (C ABI: ``include/mimo_bwd_fwd.h``); this
package only marshals arguments.
"""

from .api import MambaMimoBwdFwdOutputs, fwd_workspace_size, mamba_mimo_bwd_fwd, mamba_mimo_fwd, workspace_size

__all__ = ["MambaMimoBwdFwdOutputs", "mamba_mimo_bwd_fwd", "mamba_mimo_fwd", "workspace_size",
           "fwd_workspace_size"]
