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
  st[0] = stage_after(st[0], st[1], tag, accept, next);
  st[1] = tag;
}

// The guard's transitions, checked by the compiler on the sequences that matter (T: this
// configuration's tag, U: another's).
constexpr uint32_t T = 0x1234abcdu, U = 0x1234abceu;
constexpr uint32_t rank(uint32_t cur, uint32_t t) {
  return stage_after(cur, t, T, kAcceptDraftRank, DAP_STAGE_RANKED);
}
constexpr uint32_t attend(uint32_t cur, uint32_t t) {
  return stage_after(cur, t, T, kAcceptAttention, DAP_STAGE_ATTENDED);
}
constexpr bool restorable(uint32_t cur, uint32_t t) { return stage_ok(cur, t, T, kAcceptRestore); }
// prepare -> draft_rank -> attention -> restore, and its repeats
static_assert(stage_after(0xFFFFFFFFu, 0u, T, kStageAny, DAP_STAGE_PREPARED) == DAP_STAGE_PREPARED, "");
static_assert(rank(DAP_STAGE_PREPARED, T) == DAP_STAGE_RANKED, "");
static_assert(attend(DAP_STAGE_RANKED, T) == DAP_STAGE_ATTENDED, "");
static_assert(restorable(DAP_STAGE_ATTENDED, T), "");
static_assert(attend(DAP_STAGE_ATTENDED, T) == DAP_STAGE_ATTENDED, "");
static_assert(rank(DAP_STAGE_ATTENDED, T) == DAP_STAGE_RANKED, "");
// out of order
static_assert(rank(0u, 0u) == DAP_STAGE_BROKEN, "");
static_assert(attend(DAP_STAGE_PREPARED, T) == DAP_STAGE_BROKEN, "");
static_assert(!restorable(DAP_STAGE_RANKED, T) && !restorable(DAP_STAGE_PREPARED, T), "");
// a stage written under another configuration
static_assert(rank(DAP_STAGE_PREPARED, U) == DAP_STAGE_BROKEN, "");
static_assert(attend(DAP_STAGE_RANKED, U) == DAP_STAGE_BROKEN, "");
static_assert(!restorable(DAP_STAGE_ATTENDED, U), "");
// broken stays broken until the next prepare
static_assert(rank(DAP_STAGE_BROKEN, T) == DAP_STAGE_BROKEN, "");
static_assert(attend(DAP_STAGE_BROKEN, T) == DAP_STAGE_BROKEN && !restorable(DAP_STAGE_BROKEN, T), "");
// memory no call wrote: all-zero and all-one words, a stage number beyond the accept masks
static_assert(attend(0u, 0u) == DAP_STAGE_BROKEN && attend(0xFFFFFFFFu, T) == DAP_STAGE_BROKEN, "");
static_assert(!stage_ok(kStageMagic | 40u, T, T, 0xFFFFFFFEu), "");

}  // namespace

hipError_t launch_stage(const Geo& g, const Ws& w, uint32_t accept, uint32_t next, hipStream_t s) {
  stage_kernel<<<1, 64, 0, s>>>(w.stage, g.tag, accept, next);
  return hipGetLastError();
}

}  // namespace dap
