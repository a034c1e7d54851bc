// Per-head ranking of all region pairs and 4-level block assignment (gfx950).
//
// Method: "DraftAttention2" -- pchao.org blog, section 方法概览 bullet 2 (within each head all region
// pairs are sorted by draft score; by quota they get 16-bit, then INT8, then 4-bit; the rest are
// skipped; rows may differ in count and mix under the head budget); newx.sg paper card, AI Summary
// (a shared sorting mechanism).
//
// Only the three cut keys are needed, not a full sort: the pair at rank c-1 for c in (c16, c8, c4).
// Keys are 87-bit integers, ascending key = (score descending, pair index ascending):
//   key = ((~bits(score) & 0x7fff'ffff'ffff'ffff) << 24) | (qb*Nb + kb)
// (scores are >= 0, so their IEEE bit patterns are ordered).  An MSD radix select finds each cut
// key exactly in 8 digit passes (7 x 11 bits + 10 bits); each pass is a histogram over all pairs
// whose key shares the cut's known prefix (LDS histograms, flushed with integer atomics, so the
// result does not depend on scheduling), then a one-workgroup scan per head picks the digit.
// After the first two digits (exponent and 11 mantissa bits) the pairs that still share a cut's
// prefix are few: they are compacted once into a candidate list (in the max-pool logits map, which
// is dead after the draft mix) and the remaining six passes histogram only that list.  A head whose
// candidates overflow the list keeps scanning all its pairs.
// Finally one wave per query row classifies its pairs against the cut keys, writes the uint8 map
// and the per-level key-block lists (ascending kb) with ballot/popcount compaction.
#include "dap_internal.h"

namespace dap {
namespace {

typedef unsigned __int128 u128;

__device__ __forceinline__ u128 pair_key(double score, uint32_t idx) {
  const unsigned long long u = (unsigned long long)__double_as_longlong(score);
  const unsigned long long hi = (~u) & 0x7fffffffffffffffull;
  return ((u128)hi << 24) | (u128)idx;
}

__device__ __forceinline__ u128 make_u128(unsigned long long hi, unsigned long long lo) {
  return ((u128)hi << 64) | (u128)lo;
}

__global__ void rank_init_kernel(Geo g, RankCut* st, uint32_t* hist) {
  const int bh = blockIdx.x;
  const long long cuts[3] = {g.c16, g.c8, g.c4};
  if (threadIdx.x < 3) {
    const long long c = cuts[threadIdx.x];
    RankCut r;
    r.prefix_hi = 0;
    r.prefix_lo = 0;
    r.remaining = c - 1;
    r.mode = c == 0 ? kCutNone : (c == g.pairs ? kCutAll : kCutKey);
    r.pad = 0;
    st[bh * 3 + threadIdx.x] = r;
  }
  for (int i = threadIdx.x; i < 3 * kRankBins; i += blockDim.x) hist[(size_t)bh * 3 * kRankBins + i] = 0;
}

constexpr int kHistThreads = 256;
constexpr int kPerThread = 64;
constexpr int kChunk = kHistThreads * kPerThread;
constexpr int kCompactPass = 1;  // candidates are compacted after this pass's digit is chosen

// Candidate list of one head inside its region of the max-pool logits map (pairs x 8 bytes):
// cap = pairs / 2 score bit patterns (8 bytes each) followed by cap pair indices (4 bytes each).
__device__ __forceinline__ long long cand_cap(const Geo& g) { return g.pairs / 2; }
__device__ __forceinline__ unsigned long long* cand_bits(const Geo& g, const Ws& w, int bh) {
  return reinterpret_cast<unsigned long long*>(w.lmax + (size_t)bh * g.pairs);
}
__device__ __forceinline__ uint32_t* cand_idx(const Geo& g, const Ws& w, int bh) {
  return reinterpret_cast<uint32_t*>(cand_bits(g, w, bh) + cand_cap(g));
}

__global__ __launch_bounds__(kHistThreads) void rank_hist_kernel(Geo g, Ws w, const double* __restrict__ scores,
                                                                 const RankCut* __restrict__ st,
                                                                 uint32_t* __restrict__ hist, int pass) {
  __shared__ uint32_t s_h[3][kRankBins];
  const int bh = blockIdx.y;
  bool active[3];
  u128 prefix[3];
  bool any = false;
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    const RankCut c = st[bh * 3 + j];
    active[j] = c.mode == kCutKey;
    prefix[j] = make_u128(c.prefix_hi, c.prefix_lo);
    any |= active[j];
  }
  if (!any) return;
  // Cuts that share a prefix (all three on the first pass) share one histogram: src[j] is the
  // first active cut with cut j's prefix.  The scores of a head cluster in few top-digit bins, so
  // every avoided LDS atomic is a contended one.
  int src[3];
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    src[j] = j;
#pragma unroll
    for (int k = 0; k < j; ++k)
      if (src[j] == j && active[k] && active[j] && prefix[k] == prefix[j]) src[j] = k;
  }
  // candidate mode: after the compaction, unless this head's list overflowed
  const long long ncand = pass > kCompactPass ? (long long)st[bh * 3].pad : -1;
  const bool cand = ncand >= 0 && ncand <= cand_cap(g);
  const unsigned long long* cb = cand_bits(g, w, bh);
  const uint32_t* ci = cand_idx(g, w, bh);
  const long long n = cand ? ncand : (long long)g.pairs;
  const long long i0 = (long long)blockIdx.x * kChunk;
  if (i0 >= n) return;  // uniform per workgroup
  const long long i1 = min(n, i0 + kChunk);
  for (int i = threadIdx.x; i < 3 * kRankBins; i += kHistThreads) (&s_h[0][0])[i] = 0;
  __syncthreads();
  const int shift = rank_digit_shift(pass);
  const int top = shift + rank_digit_width(pass);
  const uint32_t mask = (1u << rank_digit_width(pass)) - 1u;
  const double* sc = scores + (size_t)bh * g.pairs;
  for (long long i = i0 + threadIdx.x; i < i1; i += kHistThreads) {
    const u128 key = cand ? pair_key(__longlong_as_double((long long)cb[i]), ci[i])
                          : pair_key(sc[i], (uint32_t)i);
    const u128 hi = key >> top;
    const uint32_t digit = (uint32_t)(key >> shift) & mask;
#pragma unroll
    for (int j = 0; j < 3; ++j)
      if (active[j] && src[j] == j && hi == prefix[j]) atomicAdd(&s_h[j][digit], 1u);
  }
  __syncthreads();
  uint32_t* gh = hist + (size_t)bh * 3 * kRankBins;
  for (int i = threadIdx.x; i < 3 * kRankBins; i += kHistThreads) {
    const int j = i / kRankBins;
    const uint32_t v = s_h[src[j]][i - j * kRankBins];
    if (active[j] && v) atomicAdd(&gh[i], v);
  }
}

// Appends every pair whose key shares an active cut's prefix (known after pass kCompactPass) to
// the head's candidate list.  Slots come from one atomic per wave, so the list order depends on
// scheduling; the histograms that read it do not.  The count keeps growing past the capacity, which
// tells later passes that the list overflowed.
__global__ __launch_bounds__(kHistThreads) void rank_compact_kernel(Geo g, Ws w, const double* __restrict__ scores,
                                                                    RankCut* __restrict__ st) {
  const int bh = blockIdx.y;
  bool active[3];
  u128 prefix[3];
  bool any = false;
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    const RankCut c = st[bh * 3 + j];
    active[j] = c.mode == kCutKey;
    prefix[j] = make_u128(c.prefix_hi, c.prefix_lo);
    any |= active[j];
  }
  if (!any) return;
  const int top = rank_digit_shift(kCompactPass);  // bits below the known prefix
  const double* sc = scores + (size_t)bh * g.pairs;
  unsigned long long* cb = cand_bits(g, w, bh);
  uint32_t* ci = cand_idx(g, w, bh);
  const long long cap = cand_cap(g);
  int* counter = &st[bh * 3].pad;
  const int lane = threadIdx.x & 63;
  const unsigned long long below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  const long long i0 = (long long)blockIdx.x * kChunk;
  const long long i1 = min((long long)g.pairs, i0 + kChunk);
  for (long long b0 = i0; b0 < i1; b0 += kHistThreads) {  // same trip count for every lane
    const long long i = b0 + threadIdx.x;
    bool hit = false;
    unsigned long long bits = 0;
    if (i < i1) {
      const double v = sc[i];
      bits = (unsigned long long)__double_as_longlong(v);
      const u128 hi = pair_key(v, (uint32_t)i) >> top;
#pragma unroll
      for (int j = 0; j < 3; ++j) hit |= active[j] && hi == prefix[j];
    }
    const unsigned long long m = __ballot(hit);
    if (m) {
      int wbase = 0;
      if (lane == 0) wbase = atomicAdd(counter, __popcll(m));
      wbase = __shfl(wbase, 0);
      if (hit) {
        const long long slot = (long long)wbase + __popcll(m & below);
        if (slot < cap) {
          cb[slot] = bits;
          ci[slot] = (uint32_t)i;
        }
      }
    }
  }
}

// One workgroup per head: choose the digit of each active cut and clear the histograms.
__global__ __launch_bounds__(256) void rank_select_kernel(RankCut* st, uint32_t* hist, int pass) {
  __shared__ unsigned long long s_scan[256];
  __shared__ int s_digit;
  __shared__ long long s_rem;
  const int bh = blockIdx.x, tid = threadIdx.x;
  constexpr int per = kRankBins / 256;  // 8 bins per thread
  const int width = rank_digit_width(pass);
  for (int j = 0; j < 3; ++j) {
    RankCut c = st[bh * 3 + j];  // uniform
    uint32_t* h = hist + ((size_t)bh * 3 + j) * kRankBins;
    if (c.mode == kCutKey) {
      unsigned long long cnt[per];
      unsigned long long tsum = 0;
#pragma unroll
      for (int b = 0; b < per; ++b) {
        cnt[b] = h[tid * per + b];
        tsum += cnt[b];
      }
      s_scan[tid] = tsum;
      __syncthreads();
      // inclusive Hillis-Steele scan over 256 thread sums
      for (int o = 1; o < 256; o <<= 1) {
        const unsigned long long add = tid >= o ? s_scan[tid - o] : 0ull;
        __syncthreads();
        s_scan[tid] += add;
        __syncthreads();
      }
      const unsigned long long base = s_scan[tid] - tsum;
      const long long t = c.remaining;
      if ((long long)base <= t && t < (long long)(base + tsum)) {
        unsigned long long cum = base;
#pragma unroll
        for (int b = 0; b < per; ++b) {
          if ((long long)(cum + cnt[b]) > t) {
            s_digit = tid * per + b;
            s_rem = t - (long long)cum;
            break;
          }
          cum += cnt[b];
        }
      }
      __syncthreads();
      if (tid == 0) {
        u128 p = make_u128(c.prefix_hi, c.prefix_lo);
        p = (p << width) | (u128)(uint32_t)s_digit;
        c.prefix_hi = (unsigned long long)(p >> 64);
        c.prefix_lo = (unsigned long long)p;
        c.remaining = s_rem;
        st[bh * 3 + j] = c;
      }
      __syncthreads();
    }
#pragma unroll
    for (int b = 0; b < per; ++b) h[tid * per + b] = 0;
  }
}

// One wave per query row: level of each pair, uint8 map, per-level ascending kb lists, counts.
__global__ __launch_bounds__(256) void rank_assign_kernel(Geo g, const double* __restrict__ scores,
                                                         const RankCut* __restrict__ st, uint8_t* __restrict__ map,
                                                         uint16_t* __restrict__ lists, int32_t* __restrict__ counts) {
  const int lane = threadIdx.x & 63;
  const int qb = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int bh = blockIdx.y;
  if (qb >= g.Nb) return;
  int mode[3];
  u128 cut[3];
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    const RankCut c = st[bh * 3 + j];
    mode[j] = c.mode;
    cut[j] = make_u128(c.prefix_hi, c.prefix_lo);
  }
  const int Nb = g.Nb;
  const size_t rowoff = (size_t)bh * g.pairs + (size_t)qb * Nb;
  const double* sc = scores + rowoff;
  auto level_of = [&](int kb) -> int {
    const u128 key = pair_key(sc[kb], (uint32_t)((size_t)qb * Nb + kb));
    int lv = 0;
#pragma unroll
    for (int j = 2; j >= 0; --j) {  // j = 0: 16-bit cut, 1: 8-bit, 2: 4-bit
      const bool in = mode[j] == kCutAll || (mode[j] == kCutKey && key <= cut[j]);
      if (in) lv = 3 - j;
    }
    return lv;
  };
  const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int n[4] = {0, 0, 0, 0};
  for (int kb0 = 0; kb0 < Nb; kb0 += 64) {
    const int kb = kb0 + lane;
    const int lv = kb < Nb ? level_of(kb) : -1;
    if (kb < Nb) map[rowoff + kb] = (uint8_t)lv;
#pragma unroll
    for (int L = 1; L <= 3; ++L) n[L] += __popcll(__ballot(lv == L));
  }
  uint16_t* lst = lists + rowoff;
  int base[4] = {0, n[3] + n[2], n[3], 0};  // offsets of the 4-bit, 8-bit, 16-bit lists
  for (int kb0 = 0; kb0 < Nb; kb0 += 64) {
    const int kb = kb0 + lane;
    const int lv = kb < Nb ? level_of(kb) : -1;
#pragma unroll
    for (int L = 1; L <= 3; ++L) {
      const unsigned long long m = __ballot(lv == L);
      if (lv == L) lst[base[L] + __popcll(m & below)] = (uint16_t)kb;
      base[L] += __popcll(m);
    }
  }
  if (lane == 0) {
    int32_t* cnt = counts + ((size_t)bh * Nb + qb) * 4;
    cnt[0] = n[3];
    cnt[1] = n[2];
    cnt[2] = n[1];
    cnt[3] = 0;
  }
}


// Attention work order for one head (one workgroup): the head's query blocks are ranked by cost
// (3 per 16-bit pair, 2 per low-bit pair; ties by row) and dealt to the 8 accelerator dies in
// snake order, so that each die's share of the head holds rows of every length and about an
// eighth of the work.  A die runs its rows most expensive first, so long rows do not trail at the
// end of the launch.  (Contiguous row ranges per die kept neighbouring rows on one die's L2 but
// left the dies up to 6 % apart in work; clustering rows with similar key lists onto a die raised
// its L2 hit rate but made co-resident workgroups request the same tiles at the same moment.)
constexpr int kOrderThreads = 1024;

__device__ void bitonic_sort_u64(unsigned long long* a, int n_pow2) {
  for (int k = 2; k <= n_pow2; k <<= 1)
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < n_pow2; i += blockDim.x) {
        const int ixj = i ^ j;
        if (ixj > i) {
          const unsigned long long x = a[i], y = a[ixj];
          const bool up = (i & k) == 0;
          if ((x > y) == up) {
            a[i] = y;
            a[ixj] = x;
          }
        }
      }
      __syncthreads();
    }
}

__global__ __launch_bounds__(kOrderThreads) void rank_order_kernel(Geo g,
                                                                  const int32_t* __restrict__ counts,
                                                                  uint32_t* __restrict__ order) {
  __shared__ unsigned long long s_key[4096];
  const int bh = blockIdx.x, Nb = g.Nb;
  int n2 = 1;
  while (n2 < Nb) n2 <<= 1;
  // key: (descending cost, row); padding keys sort last
  for (int qb = threadIdx.x; qb < n2; qb += blockDim.x) {
    unsigned long long key = ~0ull;
    if (qb < Nb) {
      const int32_t* cnt = counts + ((size_t)bh * Nb + qb) * 4;
      const int cost = 3 * cnt[0] + 2 * (cnt[1] + cnt[2]);  // <= 3 * 4096
      key = ((unsigned long long)(16383 - cost) << 16) | (unsigned)qb;
    }
    s_key[qb] = key;
  }
  __syncthreads();
  bitonic_sort_u64(s_key, n2);
  const int stride = xcd_stride(g.bh, Nb);
  for (int i = threadIdx.x; i < Nb; i += blockDim.x) {
    const int qb = (int)(s_key[i] & 0xffff);
    const int x = xcd_die_of_rank(i);
    order[(size_t)x * stride + (size_t)bh * xcd_chunk_size(x, Nb) + i / kXcds] = ((uint32_t)bh << 16) | (uint32_t)qb;
  }
}

}  // namespace

hipError_t launch_rank(const Geo& g, const Ws& w, hipStream_t s) {
  RankCut* st = static_cast<RankCut*>(w.rank_state);
  rank_init_kernel<<<g.bh, 256, 0, s>>>(g, st, w.rank_hist);
  const unsigned chunks = (unsigned)((g.pairs + kChunk - 1) / kChunk);
  for (int pass = 0; pass < kRankDigits; ++pass) {
    rank_hist_kernel<<<dim3(chunks, g.bh), kHistThreads, 0, s>>>(g, w, w.scores, st, w.rank_hist, pass);
    rank_select_kernel<<<g.bh, 256, 0, s>>>(st, w.rank_hist, pass);
    if (pass == kCompactPass)
      rank_compact_kernel<<<dim3(chunks, g.bh), kHistThreads, 0, s>>>(g, w, w.scores, st);
  }
  rank_assign_kernel<<<dim3((g.Nb + 3) / 4, g.bh), 256, 0, s>>>(g, w.scores, st, w.map, w.lists,
                                                                   w.counts);
  rank_order_kernel<<<g.bh, kOrderThreads, 0, s>>>(g, w.counts, w.order);
  return hipGetLastError();
}

}  // namespace dap
