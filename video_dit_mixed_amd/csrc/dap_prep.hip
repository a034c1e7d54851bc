// Operand preparation (gfx950): region reorder + padding, avg/max pooling, INT8 and MXFP4
// quantisation of Q and K in one pass over each tensor; V absmax, then V reorder + transpose +
// pack into the bf16 and FP8 matrix-core layouts.
//
// Method: "DraftAttention2" -- pchao.org blog, section 方法概览 bullet 4 (the reorder, the pooling
// and the Q/K quantisation are done in the same preparation pass) and the Figure 3 caption (each
// spatial region becomes one run of consecutive rows, padded where the frame ends; V is reordered
// and transposed while its operands are packed).  Pooling: section 方法概览 bullet 1 (one mean and
// one per-channel maximum per region).
//
// Number formats (exact, so codes match a reference bit for bit):
//   INT8 per (head, block):   a = max|x| over the block, r = 127/a (fp32, correctly rounded),
//                             code = clamp(rne(x*r), -127, 127), scale = a/127; a = 0, or r
//                             overflowing to infinity (a below about 3.7e-37) -> all 0.
//   MXFP4 per (row, 32 ch):   e = clamp(floor(log2 amax) - 2, -127, 127) (amax = 0 -> -127),
//                             byte = e + 127, code = E2M1 rne saturating of x*2^-e, sign = sign
//                             bit of x; two codes per byte, even channel in the low nibble.
//   FP8 V per (head, ch):     a_d = max|V[:, d]| over real tokens, r = 448/a_d,
//                             code = e4m3fn rne of x*r (|x*r| <= 448, so no saturation case;
//                             the hardware converter v_cvt_pk_fp8_f32), scale = a_d/448; a_d = 0,
//                             or r overflowing (a_d below about 1.3e-36) -> codes 0, scale 0.
//   NVFP4 per (head, tensor) and (row, 16 ch), when selected instead of MXFP4 (the pages'
//                             example 4-bit format, blog section 方法概览 bullet 2):
//                             t = amax/2688 over the head's tensor (per-channel maxima from
//                             v_amax_kernel, then their maximum), d = 6 t, scale byte =
//                             e4m3fn rne of a_16 / d (hardware converter), step = scale x t,
//                             inv = 1/step (0 if step is 0 or inv overflows), code = E2M1 of
//                             |x| x inv with the sign bit of x; t = 0 -> every code and scale 0.
//                             Also written: E2M1 value x scale as bf16 (exact: at most 6
//                             significant bits), the operand of the 4-bit Q K^T.
// Launch shapes: prep_qk one 256-thread workgroup per (block, head, tensor); v_amax a grid of
// token slices per head; v_pack one workgroup per (block, head).  Reads are whole region rows
// (region_w * D * 2 contiguous bytes) with 16-byte lanes, marked non-temporal: each input byte is
// read once per pass (prepare -4 to -7 % against cached loads).
#pragma clang fp contract(off)

#include <mutex>

#include "dap_internal.h"

namespace dap {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// Unpack a 16-byte chunk of 8 bf16 values.
__device__ __forceinline__ void unpack8(const uint4& u, float (&x)[8]) {
  x[0] = bf16_to_f32(u.x & 0xffff);
  x[1] = bf16_to_f32(u.x >> 16);
  x[2] = bf16_to_f32(u.y & 0xffff);
  x[3] = bf16_to_f32(u.y >> 16);
  x[4] = bf16_to_f32(u.z & 0xffff);
  x[5] = bf16_to_f32(u.z >> 16);
  x[6] = bf16_to_f32(u.w & 0xffff);
  x[7] = bf16_to_f32(u.w >> 16);
}

// 16-byte load marked non-temporal: the inputs are read once, so they need not displace
// cached lines
__device__ __forceinline__ uint4 load_once16(const uint16_t* p) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(t.x, t.y, t.z, t.w);
}

__device__ __forceinline__ uint32_t word_of(const uint4& u, int i) {
  return i == 0 ? u.x : i == 1 ? u.y : i == 2 ? u.z : u.w;
}

// E2M1 magnitude code of |v| (round to nearest, ties to the even code, saturate at 6).
__device__ __forceinline__ uint32_t e2m1_code(float v) {
  return (uint32_t)(v > 0.25f) + (uint32_t)(v >= 0.75f) + (uint32_t)(v > 1.25f) +
         (uint32_t)(v >= 1.75f) + (uint32_t)(v > 2.5f) + (uint32_t)(v >= 3.5f) +
         (uint32_t)(v > 5.0f);
}

// MX shared exponent of a group whose max magnitude is amax (a bf16 value held in fp32).
__device__ __forceinline__ int mx_exponent(float amax) {
  const uint32_t ef = (__float_as_uint(amax) >> 23) & 0xff;
  if (amax == 0.0f || ef == 0) return -127;  // zero or subnormal: floor(log2) - 2 < -127
  int e = (int)ef - 127 - 2;
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// Value of a non-negative finite e4m3fn code (exact).
__device__ __forceinline__ float e4m3_value(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  return e == 0 ? (float)m * 0.001953125f : ldexpf((float)(8u + m), (int)e - 10);
}

// Value of an E2M1 magnitude code 0..7: 0, 0.5, 1, 1.5, 2, 3, 4, 6.
__device__ __forceinline__ float e2m1_value(uint32_t m) {
  return m < 4u ? 0.5f * (float)m : (m == 7u ? 6.0f : (float)m - 2.0f);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

struct BlockCoord {
  int t, ry, rx, vh, vw;
};

__device__ __forceinline__ BlockCoord block_coord(const Geo& g, int b) {
  BlockCoord c;
  const int per = g.nby * g.nbx;
  c.t = b / per;
  const int rem = b - c.t * per;
  c.ry = rem / g.nbx;
  c.rx = rem - c.ry * g.nbx;
  c.vh = min(g.rh, g.H - c.ry * g.rh);
  c.vw = min(g.rw, g.W - c.rx * g.rw);
  return c;
}

// ------------------------------------------------------------------------------------ Q / K
template <int D>
__global__ __launch_bounds__(kThreads) void prep_qk_kernel(Geo g, const uint16_t* __restrict__ q,
                                                          const uint16_t* __restrict__ k, Ws w) {
  constexpr int CH = D / 8;           // 16-byte chunks per row
  constexpr int RP = kThreads / CH;   // rows per pass
  constexpr int MAXP = 128 / RP;      // passes for the largest block (128 rows)
  __shared__ double s_sum[RP][D];
  __shared__ float s_max[RP][D];
  __shared__ float s_red[kThreads / 64];

  const int b = blockIdx.x, bh = blockIdx.y, tensor = blockIdx.z;
  const uint16_t* src = (tensor == 0 ? q : k) + (size_t)bh * g.N * D;
  const int tid = threadIdx.x;
  const int c = tid % CH;
  const int r0 = tid / CH;
  const int B = g.B;
  const BlockCoord bc = block_coord(g, b);

  uint4 raw[MAXP];
  bool ok[MAXP];
  bool inblk[MAXP];
#pragma unroll
  for (int p = 0; p < MAXP; ++p) {
    const int r = r0 + p * RP;
    raw[p] = make_uint4(0, 0, 0, 0);
    ok[p] = false;
    inblk[p] = r < B;
    if (r < B) {
      const int iy = r / g.rw, ix = r - (r / g.rw) * g.rw;
      if (iy < bc.vh && ix < bc.vw) {
        const size_t n = ((size_t)bc.t * g.H + bc.ry * g.rh + iy) * g.W + bc.rx * g.rw + ix;
        raw[p] = load_once16(src + n * D + c * 8);
        ok[p] = true;
      }
    }
  }

  const size_t row0 = (size_t)bh * g.Np + (size_t)b * B;  // first packed row of this block

  // bf16 packed copy
  if (g.need16) {
    uint16_t* dst = tensor == 0 ? w.q_bf16 : w.k_bf16;
#pragma unroll
    for (int p = 0; p < MAXP; ++p)
      if (inblk[p])
        *reinterpret_cast<uint4*>(dst + (row0 + r0 + p * RP) * D + c * 8) = raw[p];
  }

  // per-thread partial pooling and block absmax
  double psum[8];
  float pmax[8];
  float amax = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    psum[j] = 0.0;
    pmax[j] = -INFINITY;
  }
#pragma unroll
  for (int p = 0; p < MAXP; ++p) {
    float x[8];
    unpack8(raw[p], x);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      amax = fmaxf(amax, fabsf(x[j]));
      if (ok[p]) {
        psum[j] += (double)x[j];
        pmax[j] = fmaxf(pmax[j], x[j]);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    s_sum[r0][c * 8 + j] = psum[j];
    s_max[r0][c * 8 + j] = pmax[j];
  }
  amax = wave_max(amax);
  if ((tid & 63) == 0) s_red[tid >> 6] = amax;
  __syncthreads();
  amax = s_red[0];
#pragma unroll
  for (int i = 1; i < kThreads / 64; ++i) amax = fmaxf(amax, s_red[i]);

  // pooled descriptors: channel d = tid (fixed summation order over the RP partials)
  if (tid < D) {
    double s = 0.0;
    float m = -INFINITY;
    for (int i = 0; i < RP; ++i) {
      s += s_sum[i][tid];
      m = fmaxf(m, s_max[i][tid]);
    }
    const size_t o = ((size_t)bh * g.Nb + b) * D + tid;
    const double nvalid = (double)(bc.vh * bc.vw);
    if (tensor == 0) {
      w.q_avg[o] = s / nvalid;
      w.q_max[o] = (double)m;
    } else {
      w.k_avg[o] = s / nvalid;
      w.k_max[o] = (double)m;
    }
  }

  // INT8 per block
  if (g.need8) {
    // 127/0 is +inf as well: one test covers empty and vanishingly small blocks
    const float r_raw = 127.0f / amax;
    const bool zero_blk = !(r_raw <= 3.402823466e38f);
    const float r = zero_blk ? 0.0f : r_raw;
    int8_t* dst = tensor == 0 ? w.q_i8 : w.k_i8;
#pragma unroll
    for (int p = 0; p < MAXP; ++p) {
      if (!inblk[p]) continue;
      float x[8];
      unpack8(raw[p], x);
      uint32_t lo = 0, hi = 0;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float cv = rintf(x[j] * r);
        cv = fminf(fmaxf(cv, -127.0f), 127.0f);
        const uint32_t byte = (uint32_t)((int)cv) & 0xffu;
        if (j < 4) lo |= byte << (8 * j);
        else hi |= byte << (8 * (j - 4));
      }
      *reinterpret_cast<uint2*>(dst + (row0 + r0 + p * RP) * D + c * 8) = make_uint2(lo, hi);
    }
    if (tid == 0) {
      float* sc = tensor == 0 ? w.q_i8_scale : w.k_i8_scale;
      sc[(size_t)bh * g.Nb + b] = zero_blk ? 0.0f : amax / 127.0f;
    }
  }

  // NVFP4 per (row, 16-channel group): a group is 2 adjacent lanes (chunks 2G, 2G+1)
  if (g.need4 && g.fp4_format == DAP_FP4_NVFP4) {
    float ta = 0.0f;  // the head's tensor maximum: maximum of the per-channel maxima
    for (int ch = tid; ch < D; ch += kThreads)
      ta = fmaxf(ta, __uint_as_float(w.qk_amax[((size_t)tensor * g.bh + bh) * D + ch]));
    ta = wave_max(ta);
    __syncthreads();  // every thread has read s_red for the block maximum
    if ((tid & 63) == 0) s_red[tid >> 6] = ta;
    __syncthreads();
    ta = s_red[0];
#pragma unroll
    for (int i = 1; i < kThreads / 64; ++i) ta = fmaxf(ta, s_red[i]);
    const float t = ta / 2688.0f;
    if (b == 0 && tid == 0) w.nv_tscale[(size_t)bh * 2 + tensor] = t;
    const float d6 = 6.0f * t;
    uint8_t* dst = tensor == 0 ? w.q_fp4 : w.k_fp4;
    uint8_t* dsc = tensor == 0 ? w.q_nv_scale : w.k_nv_scale;
    uint16_t* dbf = tensor == 0 ? w.q_nv_bf16 : w.k_nv_bf16;
#pragma unroll
    for (int p = 0; p < MAXP; ++p) {
      float x[8];
      unpack8(raw[p], x);
      float ga = 0.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j) ga = fmaxf(ga, fabsf(x[j]));
      ga = fmaxf(ga, __shfl_xor(ga, 1));
      if (!inblk[p]) continue;
      uint32_t sgc = 0;
      float sgv = 0.0f, inv = 0.0f;
      if (t > 0.0f) {
        // e4m3fn, round to nearest even: a_16 / d <= 448 (1 + 2^-23), so never past 448
        sgc = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(ga / d6, 0.0f, 0, false) & 0xffu;
        sgv = e4m3_value(sgc);
        const float step = sgv * t;
        inv = step > 0.0f ? 1.0f / step : 0.0f;
        if (!(inv <= 3.402823466e38f)) inv = 0.0f;
      }
      uint32_t packed = 0;
      uint32_t bw[4] = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t sgn = t > 0.0f ? (word_of(raw[p], j >> 1) >> ((j & 1) ? 31 : 15)) & 1u : 0u;
        const uint32_t mag = e2m1_code(fabsf(x[j]) * inv);
        packed |= (mag | (sgn << 3)) << (4 * j);
        const uint32_t vb = (__float_as_uint(e2m1_value(mag) * sgv) >> 16) | (sgn << 15);
        bw[j >> 1] |= vb << (16 * (j & 1));
      }
      const size_t row = row0 + r0 + p * RP;
      *reinterpret_cast<uint32_t*>(dst + row * (D / 2) + c * 4) = packed;
      *reinterpret_cast<uint4*>(dbf + row * D + c * 8) = make_uint4(bw[0], bw[1], bw[2], bw[3]);
      if ((c & 1) == 0) dsc[row * (D / 16) + (c >> 1)] = (uint8_t)sgc;
    }
  }

  // MXFP4 per (row, 32-channel group): a group is 4 adjacent lanes (chunks 4G..4G+3)
  if (g.need4 && g.fp4_format == DAP_FP4_MXFP4) {
    uint8_t* dst = tensor == 0 ? w.q_fp4 : w.k_fp4;
    uint8_t* dse = tensor == 0 ? w.q_e8m0 : w.k_e8m0;
#pragma unroll
    for (int p = 0; p < MAXP; ++p) {
      float x[8];
      unpack8(raw[p], x);
      float ga = 0.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j) ga = fmaxf(ga, fabsf(x[j]));
      ga = fmaxf(ga, __shfl_xor(ga, 1));
      ga = fmaxf(ga, __shfl_xor(ga, 2));
      if (!inblk[p]) continue;
      const int e = mx_exponent(ga);
      uint32_t packed = 0;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t sgn = (word_of(raw[p], j >> 1) >> ((j & 1) ? 31 : 15)) & 1u;
        const uint32_t code = e2m1_code(fabsf(ldexpf(x[j], -e))) | (sgn << 3);
        packed |= code << (4 * j);
      }
      const size_t row = row0 + r0 + p * RP;
      *reinterpret_cast<uint32_t*>(dst + row * (D / 2) + c * 4) = packed;
      if ((c & 3) == 0) dse[row * (D / 32) + (c >> 2)] = (uint8_t)(e + 127);
    }
  }
}

// ------------------------------------------------------------------------------------ V absmax
template <int D>
__global__ __launch_bounds__(kThreads) void v_amax_kernel(Geo g, const uint16_t* __restrict__ v,
                                                         uint32_t* __restrict__ amax_bits,
                                                         int tokens_per_slice) {
  constexpr int CH = D / 8;
  constexpr int RP = kThreads / CH;
  __shared__ float s_max[RP][D];
  const int bh = blockIdx.y;
  const int tid = threadIdx.x, c = tid % CH, r0 = tid / CH;
  const int n0 = blockIdx.x * tokens_per_slice;
  const int n1 = min(g.N, n0 + tokens_per_slice);
  const uint16_t* src = v + (size_t)bh * g.N * D;
  float m[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) m[j] = 0.0f;
  auto fold = [&](const uint4& u) {
    float x[8];
    unpack8(u, x);
#pragma unroll
    for (int j = 0; j < 8; ++j) m[j] = fmaxf(m[j], fabsf(x[j]));
  };
  // eight rows per round: their loads are all in flight before the first maximum
  constexpr int U = 8;
  int n = n0 + r0;
  for (; n + (U - 1) * RP < n1; n += U * RP) {
    uint4 u[U];
#pragma unroll
    for (int i = 0; i < U; ++i) u[i] = load_once16(src + (size_t)(n + i * RP) * D + c * 8);
#pragma unroll
    for (int i = 0; i < U; ++i) fold(u[i]);
  }
  for (; n < n1; n += RP) fold(load_once16(src + (size_t)n * D + c * 8));
#pragma unroll
  for (int j = 0; j < 8; ++j) s_max[r0][c * 8 + j] = m[j];
  __syncthreads();
  if (tid < D) {
    float a = 0.0f;
    for (int i = 0; i < RP; ++i) a = fmaxf(a, s_max[i][tid]);
    atomicMax(&amax_bits[(size_t)bh * D + tid], __float_as_uint(a));  // a >= 0: bits are ordered
  }
}

// Position of key m of a block inside the bf16 V^T row: within each 16-key chunk the stored
// order is keys 0-3, 8-11, 4-7, 12-15 (bits 2 and 3 of m swapped).
__device__ __forceinline__ int vt16_pos(int m) {
  return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}
// Position of key m inside the FP8 V^T row: within each 64-key chunk, key
// 32a + 8b + 4g + e (a in 0..1, b in 0..3, g in 0..1, e in 0..3) sits at 32g + 16a + 4b + e.
__device__ __forceinline__ int vt8_pos(int m) {
  const int k = m & 63;
  return (m & ~63) | (((k >> 2) & 1) << 5) | (((k >> 5) & 1) << 4) | (((k >> 3) & 3) << 2) |
         (k & 3);
}
// Key held at position p of the FP8 V^T row (the inverse of vt8_pos): position 32g + 16a + 4b + e
// of a 64-key chunk holds key 32a + 8b + 4g + e.
__device__ __forceinline__ int vt8_key(int p) {
  const int k = p & 63;
  return (p & ~63) | (((k >> 4) & 1) << 5) | (((k >> 2) & 3) << 3) | (((k >> 5) & 1) << 2) |
         (k & 3);
}

// ------------------------------------------------------------------------------------ V pack
// One workgroup per (block, head).  The block's B token rows are gathered into LDS in their
// natural [key][channel] order (rows padded by 4 bytes so that reads of one channel across keys
// spread over the banks); then every thread emits whole 16-byte chunks of the transposed outputs,
// reading the chunk's keys for its channel from LDS: consecutive threads cover consecutive chunks
// of one output row, so the global stores are contiguous.  FP8 codes come from the hardware
// converter (round to nearest even; |x * r| <= 448 by construction of r, so no saturation case).
template <int D>
__global__ __launch_bounds__(kThreads) void v_pack_kernel(Geo g, const uint16_t* __restrict__ v,
                                                         Ws w) {
  constexpr int CH = D / 8;                 // 16-byte chunks per token row
  constexpr int PITCH = 2 * D + 4;          // LDS bytes per key row
  __shared__ __attribute__((aligned(16))) uint8_t s_v[128 * PITCH];
  __shared__ float s_r[D];

  const int b = blockIdx.x, bh = blockIdx.y;
  const int tid = threadIdx.x;
  const int B = g.B, kp8 = g.kp8;
  const BlockCoord bc = block_coord(g, b);
  const uint16_t* src = v + (size_t)bh * g.N * D;

  if (tid < D) {
    const float a = __uint_as_float(w.v_amax[(size_t)bh * D + tid]);
    const float r = 448.0f / a;  // +inf for a = 0 and for vanishingly small channels
    const bool zero_ch = !(r <= 3.402823466e38f);
    s_r[tid] = zero_ch ? 0.0f : r;
    if (b == 0) w.v_scale[(size_t)bh * D + tid] = zero_ch ? 0.0f : a / 448.0f;
  }
  // gather: key r of the block is region pixel (iy, ix) = (r / rw, r % rw); pad keys are 0.
  // Every load of the thread is issued before the first LDS store.
  constexpr int MAXI = 128 * CH / kThreads;  // rounds for the largest block
  uint4 raw[MAXI];
#pragma unroll
  for (int p = 0; p < MAXI; ++p) {
    const int i = tid + p * kThreads;
    const int r = i / CH, c = i % CH;
    const int iy = r / g.rw, ix = r - (r / g.rw) * g.rw;
    raw[p] = make_uint4(0, 0, 0, 0);
    if (i < B * CH && iy < bc.vh && ix < bc.vw) {
      const size_t n = ((size_t)bc.t * g.H + bc.ry * g.rh + iy) * g.W + bc.rx * g.rw + ix;
      raw[p] = load_once16(src + n * D + c * 8);
    }
  }
#pragma unroll
  for (int p = 0; p < MAXI; ++p) {
    const int i = tid + p * kThreads;
    if (i < B * CH) {
      uint32_t* dstw = reinterpret_cast<uint32_t*>(s_v + (i / CH) * PITCH + 16 * (i % CH));
      dstw[0] = raw[p].x;
      dstw[1] = raw[p].y;
      dstw[2] = raw[p].z;
      dstw[3] = raw[p].w;
    }
  }
  __syncthreads();
  auto val = [&](int key, int d) -> uint32_t {
    return *reinterpret_cast<const uint16_t*>(s_v + key * PITCH + 2 * d);
  };

  // bf16 V^T rows: output position p of row d holds key vt16_pos^-1(p) (an involution)
  if (g.need16) {
    uint16_t* dst = w.vt_bf16 + ((size_t)bh * g.Nb + b) * (size_t)D * B;
    const int cpr = B / 8;  // 16-byte chunks per output row
    for (int q = tid; q < D * cpr; q += kThreads) {
      const int d = q / cpr, cc = q - (q / cpr) * cpr;
      uint32_t wv[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        wv[j] = val(vt16_pos(8 * cc + 2 * j), d) | (val(vt16_pos(8 * cc + 2 * j + 1), d) << 16);
      *reinterpret_cast<uint4*>(dst + (size_t)d * B + 8 * cc) = make_uint4(wv[0], wv[1], wv[2], wv[3]);
    }
  }
  // e4m3 V^T rows of kp8 bytes: position p holds key vt8_key(p); keys >= B are 0
  if (g.need8 || g.need4) {
    uint8_t* dst = w.vt_fp8 + ((size_t)bh * g.Nb + b) * (size_t)D * kp8;
    const int cpr = kp8 / 16;
    for (int q = tid; q < D * cpr; q += kThreads) {
      const int d = q / cpr, cc = q - (q / cpr) * cpr;
      const float r = s_r[d];
      uint32_t wv[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float x[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int key = vt8_key(16 * cc + 4 * j + e);
          // a zero channel (r = 0) gets code +0 everywhere, not the sign of x * 0
          x[e] = key < B && r != 0.0f ? bf16_to_f32(val(key, d)) * r : 0.0f;
        }
        int word = (int)__float_as_uint(x[0]);  // any value: both halves are written below
        word = __builtin_amdgcn_cvt_pk_fp8_f32(x[0], x[1], word, false);
        word = __builtin_amdgcn_cvt_pk_fp8_f32(x[2], x[3], word, true);
        wv[j] = (uint32_t)word;
      }
      *reinterpret_cast<uint4*>(dst + (size_t)d * kp8 + 16 * cc) = make_uint4(wv[0], wv[1], wv[2], wv[3]);
    }
  }
}

__global__ void fill_u32_kernel(uint32_t* p, size_t n, uint32_t v) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = v;
}

template <int D>
hipError_t prepare_d(const Geo& g, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                     const Ws& w, hipStream_t s) {
  const int slice = 2048;
  const int slices = (g.N + slice - 1) / slice;
  const size_t na = (size_t)g.bh * D;
  if (g.need4 && g.fp4_format == DAP_FP4_NVFP4) {
    // per-channel maxima of |Q| and |K| for the NVFP4 tensor scales
    fill_u32_kernel<<<(unsigned)((2 * na + 255) / 256), 256, 0, s>>>(w.qk_amax, 2 * na, 0u);
    v_amax_kernel<D><<<dim3(slices, g.bh), kThreads, 0, s>>>(g, q, w.qk_amax, slice);
    v_amax_kernel<D><<<dim3(slices, g.bh), kThreads, 0, s>>>(g, k, w.qk_amax + na, slice);
  }
  prep_qk_kernel<D><<<dim3(g.Nb, g.bh, 2), kThreads, 0, s>>>(g, q, k, w);
  fill_u32_kernel<<<(unsigned)((na + 255) / 256), 256, 0, s>>>(w.v_amax, na, 0u);
  fill_u32_kernel<<<1, 64, 0, s>>>(reinterpret_cast<uint32_t*>(w.zeros), 64, 0u);
  v_amax_kernel<D><<<dim3(slices, g.bh), kThreads, 0, s>>>(g, v, w.v_amax, slice);
  v_pack_kernel<D><<<dim3(g.Nb, g.bh), kThreads, 0, s>>>(g, v, w);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prepare(const Geo& g, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                          const Ws& w, hipStream_t s) {
  return g.D == 64 ? prepare_d<64>(g, q, k, v, w, s) : prepare_d<128>(g, q, k, v, w, s);
}

// ------------------------------------------------------------------------------------ static scratch
// The preparation's scratch is the per-channel maxima: of |V| (written by v_amax_kernel, read by
// v_pack_kernel in the same call) and, with NVFP4, of |Q| and |K| (read by prep_qk_kernel for the
// tensor scales).  dap_prepare_static_scratch keeps them in this array instead of the caller's
// workspace: V's in words [0, bh*D), Q's and K's in [kStaticScratchWords, 3 kStaticScratchWords).
// Each device that loads the library holds its own copy until the process ends; its address on
// the current device comes from hipGetSymbolAddress, taken once per device.  In host code
// `scratch` names a host-side stand-in, never a device address.
static __device__ __align__(256) uint32_t scratch[3 * kStaticScratchWords];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
uint32_t* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t static_scratch(uint32_t** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = static_cast<uint32_t*>(p);
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_prepare_static_scratch(const Geo& g, const uint16_t* q, const uint16_t* k,
                                         const uint16_t* v, const Ws& w, hipStream_t s) {
  if ((size_t)g.bh * g.D > kStaticScratchWords) return hipErrorInvalidValue;  // checked by the caller
  uint32_t* p = nullptr;
  const hipError_t e = static_scratch(&p);
  if (e != hipSuccess) return e;
  Ws ws = w;
  // each region is cleared by prepare's own fill kernels before its maxima are taken
  ws.v_amax = p;
  ws.qk_amax = p + kStaticScratchWords;  // used only when the 4-bit level is NVFP4
  return launch_prepare(g, q, k, v, ws, s);
}

}  // namespace dap
