// How fast can gfx950's matrix cores run when their A operand comes from LDS?
//
// The attention kernel's products (S^T = K Q^T and O^T += V^T P^T) take the tile operand (K rows,
// V^T rows) from LDS, one 16-byte read per lane -- 1 KB per wave -- per 32x32x16 bf16 product,
// and the query-side operand from registers.  This program times that pattern in isolation: one
// workgroup per compute unit, of 512 threads (two waves per SIMD, as in the attention kernel) and
// then of 256 (one wave per SIMD, the occupancy a wave of 64 queries would need for its registers),
// each wave looping over products and/or LDS reads, cycles taken with s_memtime (shader clock).
//
//   registers            products only, A from registers: the matrix-core peak (32 cycles each)
//   lds_per_product      each product reads its A operand from LDS, scheduled by the compiler
//   lds_b_operand        the same with the LDS operand in the B position (A from registers)
//   lds_per_two_products one read feeds two products (two B operands), half the LDS bytes
//   lds_softmax_valu     lds_per_product plus, per product, the vector work of the attention kernel's
//                        16-bit phase per product: one exponential (two issue slots) and four other
//                        instructions, about 25 VALU cycles, in independent chains
//   lds_only             the reads alone, folded with XORs: the LDS read rate of a compute unit
//
// Prints one JSON line per pattern.  Reads are conflict-free (lane l reads 16 bytes at 16 l of a
// 1 KB run), as are the attention kernel's swizzled operand reads.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <cstdlib>

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;

constexpr int kThreads = 512;
constexpr int kSlots = 8192;  // 16-byte LDS slots: 128 KB, so one workgroup per compute unit
constexpr int kUnroll = 8;

enum Pattern { kRegisters, kLdsPerProduct, kLdsB, kLdsPerTwo, kLdsSoftmaxValu, kLdsOnly, kPatterns };
const char* const kNames[kPatterns] = {"registers", "lds_per_product", "lds_b_operand", "lds_per_two_products",
                                       "lds_softmax_valu", "lds_only"};

__device__ __forceinline__ f32x16 mma(uint4 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mma_b(uint4 a, uint4 b, f32x16 c) {  // b in the B position
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

template <int P>
__global__ __launch_bounds__(kThreads) void feed_kernel(unsigned long long* cycles, float* sink, int iters) {
  __shared__ uint4 lds[kSlots];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < kSlots; i += (int)blockDim.x) lds[i] = make_uint4(3u * i, 5u * i + 1, 7u * i + 2, 0x3f803f80u);
  __syncthreads();
  const bf16x8 b0 = __builtin_bit_cast(bf16x8, make_uint4(0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u));
  const bf16x8 b1 = __builtin_bit_cast(bf16x8, make_uint4(0x3f813f81u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u));
  const uint4 areg = make_uint4(lane, lane + 1, lane + 2, 0x3f803f80u);
  f32x16 acc[4] = {}, acc2[4] = {};
  unsigned folded = 0;
  float ch[4] = {0.25f * lane, 0.5f, -0.75f, 1.0f};  // independent vector chains (lds_softmax_valu)
  const float cs = 0.0625f, nb = -0.5f;
  const int lane_slot = wave * 64 + lane;  // < 512
  __syncthreads();
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < iters; ++it) {
    // reads at base + 512 u, u < 8: base <= 7 * 512 + 511, so every slot is at most 7679 < kSlots,
    // and each read is the base register plus a constant offset
    const int base = (it & 7) * 512 + lane_slot;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      if constexpr (P == kRegisters) {
        acc[u & 3] = mma(areg, b0, acc[u & 3]);
      } else {
        const uint4 v = lds[base + 512 * u];
        if constexpr (P == kLdsPerProduct || P == kLdsPerTwo || P == kLdsSoftmaxValu) acc[u & 3] = mma(v, b0, acc[u & 3]);
        if constexpr (P == kLdsB) acc[u & 3] = mma_b(areg, v, acc[u & 3]);
        if constexpr (P == kLdsSoftmaxValu) {
          const float e = __builtin_amdgcn_exp2f(fmaf(ch[u & 3], cs, nb));
          ch[(u + 1) & 3] = fmaf(ch[(u + 1) & 3], 0.99f, e);
          ch[(u + 2) & 3] = fmaxf(ch[(u + 2) & 3], e);
          ch[(u + 3) & 3] = ch[(u + 3) & 3] + e;
        }
        if constexpr (P == kLdsPerTwo) acc2[u & 3] = mma(v, b1, acc2[u & 3]);
        if constexpr (P == kLdsOnly) folded ^= v.x ^ v.y ^ v.z ^ v.w;
      }
    }
  }
  __syncthreads();
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  if (tid == 0) cycles[blockIdx.x] = t1 - t0;
  float s = (float)folded + ch[0] + ch[1] + ch[2] + ch[3];
#pragma unroll
  for (int k = 0; k < 4; ++k)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[k][r] + acc2[k][r];
  sink[(size_t)blockIdx.x * kThreads + tid] = s;  // keeps every product and read live
}

template <int P>
hipError_t launch(int grid, int threads, unsigned long long* cycles, float* sink, int iters) {
  feed_kernel<P><<<grid, threads>>>(cycles, sink, iters);
  return hipGetLastError();
}

}  // namespace

int main(int argc, char** argv) {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
    std::fprintf(stderr, "no HIP device\n");
    return 1;
  }
  const int iters = argc > 1 ? std::min(std::max(std::atoi(argv[1]), 1), 1000000) : 4000;
  const int grid = cus;  // one workgroup per compute unit
  unsigned long long* d_cycles = nullptr;
  float* d_sink = nullptr;
  if (hipMalloc(&d_cycles, sizeof(unsigned long long) * grid) != hipSuccess ||
      hipMalloc(&d_sink, sizeof(float) * (size_t)grid * kThreads) != hipSuccess) {
    std::fprintf(stderr, "hipMalloc failed\n");
    return 1;
  }
  unsigned long long* h = new unsigned long long[grid];
  for (int wps = 2; wps >= 1; --wps) {  // waves per SIMD
  const int threads = 256 * wps;      // four SIMDs per compute unit
  for (int p = 0; p < kPatterns; ++p) {
    for (int rep = 0; rep < 2; ++rep) {  // the first run warms the clocks up
      hipError_t e = p == kRegisters       ? launch<kRegisters>(grid, threads, d_cycles, d_sink, iters)
                     : p == kLdsPerProduct ? launch<kLdsPerProduct>(grid, threads, d_cycles, d_sink, iters)
                     : p == kLdsB          ? launch<kLdsB>(grid, threads, d_cycles, d_sink, iters)
                     : p == kLdsPerTwo     ? launch<kLdsPerTwo>(grid, threads, d_cycles, d_sink, iters)
                     : p == kLdsSoftmaxValu ? launch<kLdsSoftmaxValu>(grid, threads, d_cycles, d_sink, iters)
                                           : launch<kLdsOnly>(grid, threads, d_cycles, d_sink, iters);
      if (e == hipSuccess) e = hipDeviceSynchronize();
      if (e != hipSuccess) {
        std::fprintf(stderr, "%s: %s\n", kNames[p], hipGetErrorString(e));
        return 1;
      }
    }
    if (hipMemcpy(h, d_cycles, sizeof(unsigned long long) * grid, hipMemcpyDeviceToHost) != hipSuccess) return 1;
    double avg = 0;
    for (int i = 0; i < grid; ++i) avg += (double)h[i];
    avg /= grid;
    // per SIMD: wps waves, kUnroll reads or products per wave and iteration (two products per
    // read in lds_per_two_products); per compute unit: 4 wps waves of 1 KB reads
    const double units = (double)wps * iters * kUnroll * (p == kLdsPerTwo ? 2 : 1);
    const double lds_bytes = p == kRegisters ? 0.0 : 4.0 * wps * iters * kUnroll * 1024;
    const double per = avg / units;
    char frac[32] = "null";  // a 32x32x16 bf16 product takes 32 cycles at the peak
    if (p != kLdsOnly) std::snprintf(frac, sizeof(frac), "%.3f", 32.0 / per);
    std::printf("{\"pattern\": \"%s\", \"waves_per_simd\": %d, \"cycles\": %.0f, \"cycles_per_%s_per_simd\": %.2f, "
                "\"matrix_core_fraction\": %s, \"lds_bytes_per_clk_per_cu\": %.1f, \"cus\": %d}\n",
                kNames[p], wps, avg, p == kLdsOnly ? "read" : "product", per, frac, lds_bytes / avg, cus);
  }
  }
  delete[] h;
  const bool freed = hipFree(d_cycles) == hipSuccess && hipFree(d_sink) == hipSuccess;
  return freed ? 0 : 1;
}
