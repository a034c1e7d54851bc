// Draft attention map (gfx950, fp64): pooled logits L = Qbar Kbar^T / sqrt(D) for the average and
// the max descriptors, row softmax over key regions, and the mix A = (1-lambda) A_avg + lambda A_max.
//
// Method: "DraftAttention2" -- pchao.org blog, section 方法概览 bullet 1 (Avg and Max draft maps
// from the region descriptors, mixed with weight lambda; lambda = 0 is average-only) and the
// Figure 2 caption.  fp64 keeps the scores exact enough that the per-head ranking (and so the block
// map) is reproducible bit for bit.
//
// Kernels: draft_logits -- a 128x128-tile fp64 GEMM per (head, map), writing L_avg into the score
// buffer and L_max into a scratch buffer; draft_mix -- one workgroup per query region row,
// exponentials staged in LDS, writes A over L_avg.
#pragma clang fp contract(off)

#include "dap_internal.h"

namespace dap {
namespace {

constexpr int kTile = 128;  // output tile edge (rows and columns of one workgroup)
constexpr int kKc = 16;     // channels staged per step

// 256 threads, each an 8 x 8 block of outputs (rows 8 ty + i; columns 2 tx + 32 jj + e, jj < 4,
// e < 2): per channel a thread reads its 8 Q values and 8 K values as four 16-byte LDS loads each
// (the K loads of 16 neighbouring threads are contiguous, so bank-conflict free) and does 64 fused
// multiply-adds.  Each output is one fma chain over the channels in ascending order.
template <int D>
__global__ __launch_bounds__(256) void draft_logits_kernel(Geo g, Ws w) {
  __shared__ __attribute__((aligned(16))) double sQ[kKc][kTile + 2];
  __shared__ __attribute__((aligned(16))) double sK[kKc][kTile + 2];
  const int bh = blockIdx.z >> 1, which = blockIdx.z & 1;
  const double* qbar = (which == 0 ? w.q_avg : w.q_max) + (size_t)bh * g.Nb * D;
  const double* kbar = (which == 0 ? w.k_avg : w.k_max) + (size_t)bh * g.Nb * D;
  double* dst = (which == 0 ? w.scores : w.lmax) + (size_t)bh * g.pairs;
  const int row0 = blockIdx.y * kTile, col0 = blockIdx.x * kTile;
  const int tid = threadIdx.x, ty = tid / 16, tx = tid % 16;
  double acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = 0.0;

  for (int d0 = 0; d0 < D; d0 += kKc) {
    // 128 rows x 16 channels of each operand: 2048 values, 8 per thread
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int e = tid + i * 256;
      const int r = e / kKc, c = e % kKc;
      const int qr = row0 + r, kr = col0 + r;
      sQ[c][r] = qr < g.Nb ? qbar[(size_t)qr * D + d0 + c] : 0.0;
      sK[c][r] = kr < g.Nb ? kbar[(size_t)kr * D + d0 + c] : 0.0;
    }
    __syncthreads();
#pragma unroll 2
    for (int c = 0; c < kKc; ++c) {
      double a[8], b[8];
#pragma unroll
      for (int i = 0; i < 8; i += 2) {
        const double2 qa = *reinterpret_cast<const double2*>(&sQ[c][8 * ty + i]);
        const double2 kb = *reinterpret_cast<const double2*>(&sK[c][2 * tx + 16 * i]);
        a[i] = qa.x;
        a[i + 1] = qa.y;
        b[i] = kb.x;
        b[i + 1] = kb.y;
      }
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = fma(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
  const double inv_sq = 1.0 / sqrt((double)D);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = row0 + 8 * ty + i;
    if (r >= g.Nb) continue;
    double* drow = dst + (size_t)r * g.Nb;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int col = col0 + 2 * tx + 16 * (j & ~1) + (j & 1);  // b[j] of column 2 tx + 32 (j/2) + j%2
      if (col < g.Nb) drow[col] = acc[i][j] * inv_sq;
    }
  }
}

__device__ double block_reduce(double v, bool is_max, double* s_red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const double u = __shfl_xor(v, o);
    v = is_max ? fmax(v, u) : v + u;
  }
  const int wv = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) s_red[wv] = v;
  __syncthreads();
  double r = s_red[0];
  for (int i = 1; i < (int)(blockDim.x >> 6); ++i) r = is_max ? fmax(r, s_red[i]) : r + s_red[i];
  return r;
}

__global__ __launch_bounds__(256) void draft_mix_kernel(Geo g, Ws w) {
  extern __shared__ double s_e[];  // [2][Nb]
  __shared__ double s_red[4];
  const int qb = blockIdx.x, bh = blockIdx.y;
  const int Nb = g.Nb;
  double* La = w.scores + (size_t)bh * g.pairs + (size_t)qb * Nb;
  const double* Lm = w.lmax + (size_t)bh * g.pairs + (size_t)qb * Nb;
  double* ea = s_e;
  double* em = s_e + Nb;
  double ma = -INFINITY, mm = -INFINITY;
  for (int j = threadIdx.x; j < Nb; j += blockDim.x) {
    const double a = La[j], m = Lm[j];
    ea[j] = a;
    em[j] = m;
    ma = fmax(ma, a);
    mm = fmax(mm, m);
  }
  ma = block_reduce(ma, true, s_red);
  mm = block_reduce(mm, true, s_red);
  double sa = 0.0, sm = 0.0;
  for (int j = threadIdx.x; j < Nb; j += blockDim.x) {
    const double a = exp(ea[j] - ma), m = exp(em[j] - mm);
    ea[j] = a;
    em[j] = m;
    sa += a;
    sm += m;
  }
  sa = block_reduce(sa, false, s_red);
  sm = block_reduce(sm, false, s_red);
  const double lam = g.lambda, oml = 1.0 - g.lambda;
  const double ra = 1.0 / sa, rm = 1.0 / sm;
  for (int j = threadIdx.x; j < Nb; j += blockDim.x) La[j] = oml * (ea[j] * ra) + lam * (em[j] * rm);
}

template <int D>
hipError_t draft_d(const Geo& g, const Ws& w, hipStream_t s) {
  const int nt = (g.Nb + kTile - 1) / kTile;
  draft_logits_kernel<D><<<dim3(nt, nt, 2 * g.bh), 256, 0, s>>>(g, w);
  draft_mix_kernel<<<dim3(g.Nb, g.bh), 256, 2 * g.Nb * sizeof(double), s>>>(g, w);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_draft(const Geo& g, const Ws& w, hipStream_t s) {
  return g.D == 64 ? draft_d<64>(g, w, s) : draft_d<128>(g, w, s);
}

}  // namespace dap
