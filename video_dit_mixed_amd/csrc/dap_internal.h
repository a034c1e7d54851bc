// Internal definitions shared by the libdap translation units (host launchers + gfx950 kernels).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dap.h"

namespace dap {

// Everything a kernel needs to know about one layer, passed by value.
struct Geo {
  int bh, heads, D;
  int T, H, W, rh, rw;
  int Hp, Wp, nby, nbx, Nb, B, Np, kp8;
  int N;
  long long pairs, c16, c8, c4;
  double lambda;
  int need16, need8, need4;  // does any pair use this precision
  int fp4_format;            // DAP_FP4_*
  uint32_t tag;              // configuration tag kept beside the stage word
};

// Device pointers to the workspace sections.
struct Ws {
  uint16_t* q_bf16;
  uint16_t* k_bf16;
  uint16_t* vt_bf16;
  int8_t* q_i8;
  int8_t* k_i8;
  float* q_i8_scale;
  float* k_i8_scale;
  uint8_t* q_fp4;
  uint8_t* k_fp4;
  uint8_t* q_e8m0;
  uint8_t* k_e8m0;
  uint8_t* vt_fp8;
  float* v_scale;
  uint32_t* v_amax;
  double* q_avg;
  double* q_max;
  double* k_avg;
  double* k_max;
  double* scores;
  double* lmax;
  void* rank_state;
  uint32_t* rank_hist;
  uint8_t* map;
  uint16_t* lists;
  int32_t* counts;
  uint16_t* out;
  uint8_t* zeros;
  uint32_t* order;
  uint32_t* stage;  // [0] stage word (DAP_STAGE_*), [1] configuration tag
  uint8_t* q_nv_scale;   // NVFP4 (fp4_format DAP_FP4_NVFP4): e4m3 scale per 16 channels
  uint8_t* k_nv_scale;
  uint16_t* q_nv_bf16;   // NVFP4 values without the tensor scale, as bf16 (exact)
  uint16_t* k_nv_bf16;
  float* nv_tscale;      // [bh][2]: tensor scales of Q and K
  uint32_t* qk_amax;     // [2][bh][D]: per-channel |Q| and |K| maxima (fp32 bits)
};

// Stage words: DAP_STAGE_* = kStageMagic | stage number; `accept` masks of launch_stage are sets
// of stage numbers (bit n = stage n accepted), kStageAny accepts anything (dap_prepare).
constexpr uint32_t kStageMagic = 0xDA900000u;
constexpr uint32_t kStageMagicMask = 0xFFFFFF00u;
constexpr uint32_t kStageAny = 0xFFFFFFFFu;
constexpr uint32_t stage_bit(uint32_t stage) { return 1u << (stage & 0xffu); }

// True when the stage words (cur, t) show the result of the calls this one depends on: a stage in
// `accept`, written under this configuration's tag.
__host__ __device__ constexpr bool stage_ok(uint32_t cur, uint32_t t, uint32_t tag, uint32_t accept) {
  return accept == kStageAny ||
         (t == tag && (cur & kStageMagicMask) == kStageMagic && (cur & 0xffu) < 32u &&
          ((accept >> (cur & 0xffu)) & 1u) != 0u);
}
// The word a call leaves behind: its own stage when the words showed an accepted one, else BROKEN.
__host__ __device__ constexpr uint32_t stage_after(uint32_t cur, uint32_t t, uint32_t tag,
                                                   uint32_t accept, uint32_t next) {
  return stage_ok(cur, t, tag, accept) ? next : (uint32_t)DAP_STAGE_BROKEN;
}
// What each call requires (dap_prepare accepts anything: kStageAny).
constexpr uint32_t kAcceptDraftRank =
    stage_bit(DAP_STAGE_PREPARED) | stage_bit(DAP_STAGE_RANKED) | stage_bit(DAP_STAGE_ATTENDED);
constexpr uint32_t kAcceptAttention = stage_bit(DAP_STAGE_RANKED) | stage_bit(DAP_STAGE_ATTENDED);
constexpr uint32_t kAcceptRestore = stage_bit(DAP_STAGE_ATTENDED);

// Ranking: an 87-bit key per pair, ascending key = (score descending, pair index ascending):
//   key = ((~bits(score) & 0x7fff'ffff'ffff'ffff) << 24) | pair_index, pair_index < 2^24.
// The cut of each level is found by an MSD radix select with 8 digits (7 x 11 bits + 10 bits).
constexpr int kXcds = 8;  // MI355X: 8 accelerator dies, workgroups dispatched round-robin

// Attention work slices: a head's rows, ranked by cost (most expensive first), are dealt to the
// dies in snake order (rank i goes to die i % 8 in even rounds i / 8, to die 7 - i % 8 in odd
// ones), so every die gets rows of every length and near-equal work.  Die x holds
// xcd_chunk_size(x, Nb) rows of each head: one per round, plus one from the final partial round.
__host__ __device__ inline int xcd_die_of_rank(int i) {
  const int r = i / kXcds, p = i % kXcds;
  return (r & 1) ? kXcds - 1 - p : p;
}
__host__ __device__ inline int xcd_chunk_size(int x, int Nb) {
  const int q = Nb / kXcds, rem = Nb % kXcds;
  const bool extra = (q & 1) ? (x >= kXcds - rem) : (x < rem);
  return q + (extra ? 1 : 0);
}
__host__ __device__ inline int xcd_stride(int bh, int Nb) { return bh * ((Nb + kXcds - 1) / kXcds); }

constexpr int kRankDigits = 8;
constexpr int kRankBins = 2048;
enum RankMode : int { kCutNone = 0, kCutAll = 1, kCutKey = 2 };
struct RankCut {
  unsigned long long prefix_hi;  // key bits known so far (a 128-bit integer, hi/lo halves)
  unsigned long long prefix_lo;
  long long remaining;           // rank still to skip inside the current prefix bucket
  int mode;
  int pad;
};

__host__ __device__ constexpr int rank_digit_width(int k) { return k == kRankDigits - 1 ? 10 : 11; }
// bits below digit k: 76, 65, 54, 43, 32, 21, 10, 0
__host__ __device__ constexpr int rank_digit_shift(int k) {
  return k == kRankDigits - 1 ? 0 : 87 - 11 * (k + 1);
}

// Launchers (each returns hipGetLastError() of its launches).
hipError_t launch_prepare(const Geo& g, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                          const Ws& w, hipStream_t s);
hipError_t launch_draft(const Geo& g, const Ws& w, hipStream_t s);
hipError_t launch_rank(const Geo& g, const Ws& w, hipStream_t s);
hipError_t launch_attention(const Geo& g, const Ws& w, hipStream_t s);
// the same attention, summing shader-clock cycles per part of the key-block loop into clk
// (4 phases x 8 counters, see dap_attention_section_clocks)
hipError_t launch_attention_clocked(const Geo& g, const Ws& w, unsigned long long* clk, hipStream_t s);
hipError_t launch_restore(const Geo& g, const Ws& w, uint16_t* out, hipStream_t s);
hipError_t launch_stage(const Geo& g, const Ws& w, uint32_t accept, uint32_t next, hipStream_t s);

// dap_prepare_static_scratch: the channel maxima of V (and of Q and K with NVFP4) live in a static
// device array of three regions of this many 32-bit words (768 KiB per device), so
// batch * heads * head_dim may not exceed it.
constexpr size_t kStaticScratchWords = 65536;
hipError_t launch_prepare_static_scratch(const Geo& g, const uint16_t* q, const uint16_t* k,
                                         const uint16_t* v, const Ws& w, hipStream_t s);

}  // namespace dap
