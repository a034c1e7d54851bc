// Call-order guard of one workspace (gfx950).
//
// The four calls of a layer only make sense in the order reorder/pack -> draft + rank -> attention
// -> restore (pith.science, "DraftAttention: Fast Video Diffusion via Low-Resolution Attention
// Guidance", Abstract: tokens are reordered, attended and put back).  Each call ends with a
// one-thread kernel that moves the workspace's stage word to its own stage when the word shows
// the stage it requires, and to DAP_STAGE_BROKEN otherwise; a second word holds a tag of the
// configuration that wrote it, so a stage left behind by another configuration does not count.
// Attention and restore read both words before touching anything the earlier calls wrote and
// produce zeros when they do not match (see dap_attn.hip and dap_restore.hip).
#include "dap_internal.h"

namespace dap {
namespace {

__global__ void stage_kernel(uint32_t* st, uint32_t tag, uint32_t accept, uint32_t next) {
  if (blockIdx.x != 0 || threadIdx.x != 0) return;
  const bool ok = stage_ok(st[0], st[1], tag, accept);
  st[0] = ok ? next : (uint32_t)DAP_STAGE_BROKEN;
  st[1] = tag;
}

}  // namespace

hipError_t launch_stage(const Geo& g, const Ws& w, uint32_t accept, uint32_t next, hipStream_t s) {
  stage_kernel<<<1, 64, 0, s>>>(w.stage, g.tag, accept, next);
  return hipGetLastError();
}

}  // namespace dap
