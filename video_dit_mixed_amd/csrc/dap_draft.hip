// Draft attention map (gfx950, fp64): pooled logits L = Qbar Kbar^T / sqrt(D) for the average and
// the max descriptors, row softmax over key regions, and the mix A = (1-lambda) A_avg + lambda A_max.
//
// Method: "DraftAttention2" -- pchao.org blog, section 方法概览 bullet 1 (Avg and Max draft maps
// from the region descriptors, mixed with weight lambda; lambda = 0 is average-only) and the
// Figure 2 caption.  fp64 keeps the scores exact enough that the per-head ranking (and so the block
// map) is reproducible bit for bit.
//
// Kernels: draft_logits -- a 128x128-tile fp64 GEMM per (head, map) on the fp64 matrix cores,
// writing L_avg into the score buffer and L_max into a scratch buffer; draft_mix -- one workgroup
// per query region row, exponentials staged in LDS, writes A over L_avg.
#pragma clang fp contract(off)

#include "dap_internal.h"

namespace dap {
namespace {

constexpr int kTile = 128;  // output tile edge (rows and columns of one workgroup)
constexpr int kKc = 16;     // channels staged per step
constexpr int kPitch = kKc + 2;  // LDS row pitch in doubles (see the fragment reads below)

typedef __attribute__((ext_vector_type(4))) double f64x4;

// fp64 matrix cores (v_mfma_f64_16x16x4_f64): 4 waves, wave (wr, wc) owns the 64 x 64 outputs
// rows 64 wr.., columns 64 wc.. of the tile as 4 x 4 MFMA tiles of 16 x 16.  Per 4 channels an
// MFMA takes A[m][k] = Qbar[row m][channel k] from lane m + 16 k and B[k][n] = Kbar[col n][channel
// k] from lane n + 16 k, and accumulates D[m][n] = sum_k A[m][k] B[k][n] in fp64; lane l holds
// D[4 e + l / 16][l % 16] in element e.  Operands are staged through LDS in row-major tiles with a
// pitch of 18 doubles: the 16 rows x 2 channels of a half-wave read land in 32 distinct bank pairs.
// The products of each MFMA are accumulated in channel order with fused multiply-adds, so every
// logit equals one fma chain over the channels in ascending order (measured bit for bit against a
// vector-FMA version of this kernel).  The next 16 channels are fetched into registers while the
// current ones are multiplied.  Two waves per SIMD: 214 VGPRs.
template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void draft_logits_kernel(Geo g, Ws w) {
  __shared__ __attribute__((aligned(16))) double sQ[kTile * kPitch];
  __shared__ __attribute__((aligned(16))) double sK[kTile * kPitch];
  const int bh = blockIdx.z >> 1, which = blockIdx.z & 1;
  const double* qbar = (which == 0 ? w.q_avg : w.q_max) + (size_t)bh * g.Nb * D;
  const double* kbar = (which == 0 ? w.k_avg : w.k_max) + (size_t)bh * g.Nb * D;
  double* dst = (which == 0 ? w.scores : w.lmax) + (size_t)bh * g.pairs;
  const int row0 = blockIdx.y * kTile, col0 = blockIdx.x * kTile;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int wr = wv >> 1, wc = wv & 1;
  const int li = lane & 15, lk = lane >> 4;
  // staging: thread t copies 8 channels (one 64-byte run) of row t / 2 of each operand
  const int sr = tid >> 1, sc = 8 * (tid & 1);
  const int qr = row0 + sr, kr = col0 + sr;
  f64x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f64x4{0.0, 0.0, 0.0, 0.0};

  // the next channels' operands are loaded into registers while the current ones are multiplied
  double2 qv[4], kv[4];
  auto fetch = [&](int d0) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      qv[e] = qr < g.Nb ? *reinterpret_cast<const double2*>(qbar + (size_t)qr * D + d0 + sc + 2 * e)
                        : double2{0.0, 0.0};
      kv[e] = kr < g.Nb ? *reinterpret_cast<const double2*>(kbar + (size_t)kr * D + d0 + sc + 2 * e)
                        : double2{0.0, 0.0};
    }
  };
  fetch(0);
  for (int d0 = 0; d0 < D; d0 += kKc) {
    __syncthreads();  // every wave is done with the previous channels
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      *reinterpret_cast<double2*>(sQ + sr * kPitch + sc + 2 * e) = qv[e];
      *reinterpret_cast<double2*>(sK + sr * kPitch + sc + 2 * e) = kv[e];
    }
    __syncthreads();
    if (d0 + kKc < D) fetch(d0 + kKc);
#pragma unroll
    for (int k4 = 0; k4 < kKc; k4 += 4) {
      double a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[i] = sQ[(64 * wr + 16 * i + li) * kPitch + k4 + lk];
        b[i] = sK[(64 * wc + 16 * i + li) * kPitch + k4 + lk];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  }
  const double inv_sq = 1.0 / sqrt((double)D);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = row0 + 64 * wr + 16 * i + 4 * e + lk;
      if (r >= g.Nb) continue;
      double* drow = dst + (size_t)r * g.Nb;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int col = col0 + 64 * wc + 16 * j + li;
        if (col < g.Nb) drow[col] = acc[i][j][e] * inv_sq;
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
  auto take = [&](int j, double a, double m) {
    ea[j] = a;
    em[j] = m;
    ma = fmax(ma, a);
    mm = fmax(mm, m);
  };
  // four rounds of loads in flight per thread (the maxima are exact in any order)
  constexpr int U = 4;
  const int nt = blockDim.x;
  int j = threadIdx.x;
  for (; j + (U - 1) * nt < Nb; j += U * nt) {
    double a[U], m[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      a[u] = La[j + u * nt];
      m[u] = Lm[j + u * nt];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) take(j + u * nt, a[u], m[u]);
  }
  for (; j < Nb; j += nt) take(j, La[j], Lm[j]);
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
