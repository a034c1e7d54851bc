"""MI355X-native draft-guided mixed-precision block-sparse attention (DraftAttention2 hot path).

The compute path is the C-ABI library `libdap.so` (hand-written HIP for gfx950) reached through
`video_dit_mixed_amd.binding`; `video_dit_mixed_amd.synth` holds the seeded synthetic workloads.
Submodules are imported explicitly so that importing the package never loads the GPU library.
"""
__all__ = ["binding", "synth"]
