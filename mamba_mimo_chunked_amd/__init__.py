"""MI355X (gfx950) HIP implementation of the Mamba-3 MIMO backward first stage.

``mamba_mimo_bwd_fwd`` re-runs the chunked MIMO scan and returns the bf16
chunk entry states, the same-token qk_dot and the optional dmimo_o / dz /
dmimo_z gradients; ``mamba_mimo_fwd`` returns the layer output those
gradients belong to; the ``_fp32`` variants keep every intermediate in fp32;
``mamba3_mimo_bwd_bwd`` is the stage-2 backward that consumes the first stage's
states and qk_dot; ``mamba3_siso_fwd`` is the rank-1 (SISO) forward. The computation runs in the HIP library
``_build/libmimo_bwd_fwd.so`` (C ABI: ``include/mimo_bwd_fwd.h``); this
package only marshals arguments.
"""

from .api import (MambaMimoBwdFwdOutputs, fwd_workspace_size, mamba3_mimo_bwd_bwd, mamba3_siso_fwd,
                  mamba_mimo_bwd_fwd, mamba_mimo_bwd_fwd_fp32, mamba_mimo_bwd_fwd_noalloc, mamba_mimo_fwd,
                  mamba_mimo_fwd_fp32, workspace_size)

__all__ = ["MambaMimoBwdFwdOutputs", "mamba_mimo_bwd_fwd", "mamba_mimo_bwd_fwd_noalloc", "mamba_mimo_fwd",
           "mamba_mimo_bwd_fwd_fp32",
           "mamba_mimo_fwd_fp32", "mamba3_mimo_bwd_bwd", "mamba3_siso_fwd", "workspace_size",
           "fwd_workspace_size"]
