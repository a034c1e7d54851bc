// Mixed-precision block-sparse attention with precision phases (gfx950 matrix cores).
//
// Method: "DraftAttention2" -- newx.sg paper card, Abstract, and pchao.org blog, section 方法概览
// bullet 4: the kept blocks of all precisions are handled by a single kernel that keeps one set of
// running softmax statistics and one output accumulator per query row, converts between the
// precisions' scales where the phase changes and writes the output once; bullet 2 gives the
// precisions (16-bit, INT8, 4-bit).
//
// One workgroup per (head, query block); wave w owns queries 32w..32w+31 of the block.  For every
// kept key block, in phase order 16 -> 8 -> 4 and ascending kb inside a phase:
//   S^T = K Q^T on the matrix cores (keys are the MFMA rows, so each lane holds one query column
//         and a query's scores live in two lanes: row statistics need one cross-lane step)
//         16-bit: v_mfma_f32_32x32x16_bf16        8-bit: v_mfma_i32_32x32x32_i8 (x s_q s_k)
//         4-bit:  v_mfma_scale_f32_32x32x64_f8f6f4 with E2M1 operands and E8M0 block scales
//   online softmax in registers in the log2 domain (one running-max update per key block):
//         m' = max(m, rowmax t), alpha = 2^(m - m'), P = 2^(t - m'), l = alpha l + sum P
//   O^T += V^T P^T on the matrix cores, P converted in registers to the B operand layout:
//         16-bit: bf16(P) x bf16 V        low-bit: e4m3(2^8 P) x e4m3 V (scaled f8f6f4 MFMA)
// One fp32 accumulator serves all phases.  At the first low-bit block its channel d is converted
// to low-bit units (x 2^8 / s_V[d]); the end multiplies by s_V[d] 2^-8 and divides by l.
// Key and V tiles are staged through LDS in an XOR-swizzled layout (bank-conflict-free reads).
// For 128-token blocks the load unit writes them into LDS directly (buffer loads with an LDS
// destination), so no registers hold them on the way; smaller blocks stage them through
// registers.  Two barriers per key block: after the first, the tile's V is issued (a quarter
// after each m-tile's Q K^T products) and lands during Q K^T and the softmax; after the second,
// the next tile's K is issued and lands during the P V products.  The matrix-core operand orders were fixed when the operands were packed, so
// every LDS read is one or two 16-byte loads.
#include <type_traits>

#include "dap_internal.h"

namespace dap {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) int i32x4;
typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(16))) int i32x16;

typedef __attribute__((ext_vector_type(4))) unsigned u32x4;

constexpr float kLog2e = 1.4426950408889634f;
// Word 3 of a raw buffer resource: 32-bit data format, no swizzle, no index.
constexpr int kRsrcWord3 = 0x00020000;
constexpr int kScaleOne = 0x7f7f7f7f;  // E8M0 127 = 2^0 in every byte

template <int B, int D>
struct AttnCfg {
  static constexpr int NW = B >= 32 ? B / 32 : 1;  // waves per workgroup
  static constexpr int NT = 64 * NW;
  static constexpr int KT = B >= 32 ? B : 32;      // key slots covered by the S^T m-tiles
  static constexpr int MT = KT / 32;               // S^T m-tiles (32 keys each)
  static constexpr int DT = D / 32;                // O^T m-tiles (32 channels each)
  static constexpr int KP8 = (B + 63) / 64 * 64;   // FP8 V^T row length
  static constexpr int KBYTES = KT * 2 * D;        // largest key tile (bf16)
  static constexpr int SBYTES = 64 * NW * 4;       // room for one tile's E8M0 key scales
  static constexpr int VBYTES = (D * 2 * B > D * KP8) ? D * 2 * B : D * KP8;
  // Tiles go straight to LDS for 128-token blocks; smaller blocks (more tile bytes per flop) were
  // measured faster with the tiles staged through registers.
  static constexpr bool DIRECT = B >= 128;
  static_assert(KT * D / 32 <= SBYTES, "a tile's E8M0 key scales fit in sKs");
};

// Per-phase tile geometry.  PH = 0: bf16 K rows / bf16 V^T rows; 1: int8 K / e4m3 V^T;
// 2: E2M1 K (+ E8M0 scales) / e4m3 V^T; 3 (4-bit level in NVFP4): bf16 rows of the dequantised
// NVFP4 K / e4m3 V^T.
template <int B, int D, int PH>
struct PhaseCfg {
  using C = AttnCfg<B, D>;
  static constexpr int KRB = (PH == 0 || PH == 3) ? 2 * D : (PH == 1 ? D : D / 2);  // key row bytes
  static constexpr int KRC = KRB / 16;                                 // 16-byte chunks per row
  static constexpr int VRB = PH == 0 ? 2 * B : C::KP8;                 // V^T row bytes
  static constexpr int VRC = VRB / 16;
  static_assert(KRC <= 16 && VRC <= 16, "rows up to 256 bytes");
};

// LDS tiles are stored unpadded with the 16-byte chunks of each row XOR-swizzled so that the
// 16-lane groups of a ds_read_b128 (32 consecutive rows, one chunk each) hit distinct banks:
// physical chunk = logical chunk ^ ((row / (16 / RC)) % RC) for rows of RC chunks.
template <int RC>
__device__ __forceinline__ int swz(int row, int chunk) {
  return chunk ^ ((row / (16 / RC)) % RC);
}
// Rows 32*m + n share the swizzle of row n (32 is a multiple of 16/RC * RC), so an operand read
// is a per-lane offset plus a compile-time row-tile offset.

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
  const bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ uint4 lds16(const uint8_t* p) { return *reinterpret_cast<const uint4*>(p); }

// A query's two score lanes are l and l ^ 32.  v_permlane32_swap of a register with itself leaves
// {x[l], x[l ^ 32]} in the two results of every lane (in an order that depends on the half), so
// their max / sum is the combined value, with no LDS round trip.
__device__ __forceinline__ float halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Per-workgroup context of one (head, query block) row.
struct RowCtx {
  int bh, qb, tid, n, gh;
  bool qok;
  size_t qrow;            // packed row of this lane's query
  const uint32_t* lists;  // all key-block lists, as 32-bit words
  size_t lbase;           // index of this row's first list entry
  int nb_last;            // Nb - 1: list entries are clamped to it
};

// Entry i of the row's key-block list.  The list holds 16-bit entries; the 32-bit word holding
// entry i is read at a wave-uniform address, so it is a scalar load (a 16-bit vector load would be
// waited for with vmcnt, which also waits for every tile load in flight).
typedef __attribute__((address_space(4))) const uint32_t* const_u32_ptr;  // read-only in this kernel

__device__ __forceinline__ uint32_t uniform_load(const uint32_t* p) {
  return *reinterpret_cast<const_u32_ptr>(reinterpret_cast<uintptr_t>(p));
}

__device__ __forceinline__ int list_at(const RowCtx& c, int i) {
  const size_t e = c.lbase + (size_t)i;
  const uint32_t wv = uniform_load(c.lists + (e >> 1));
  // an entry beyond the last key block can only come from a workspace the ranking did not write
  // for this configuration; clamping keeps every tile load inside the workspace
  return min((int)((e & 1) ? (wv >> 16) : (wv & 0xffffu)), c.nb_last);
}

// Moves one key block's operand tile from global memory into LDS.  Slot s (16 bytes) of a tile of
// rows with RC chunks sits at LDS byte 16*s and holds row s / RC, logical chunk (s % RC) ^ swizzle;
// thread t fills slots t, t + NT, t + 2*NT, ...  The loads are buffer loads with a wave-uniform
// resource and a 32-bit offset per lane (a 64-bit address per lane costs more to issue); rows >=
// valid fall outside the resource's range and read as zero.
//   kDirect: the load unit writes LDS itself (buffer loads with an LDS destination).  One
//     wave-level load writes 1 KB contiguous at a wave-uniform base, lane l at base + 16 l, which
//     is why the swizzle is applied on the global side.  No registers hold the tile; completion is
//     counted by vmcnt, in issue order, and commit() does nothing.
//   otherwise: the tile is held in registers from load() until commit() stores it.
template <int ROWS, int RC, int NT, bool kDirect>
struct TileMover {
  static constexpr int N = ROWS * RC / NT;  // 16-byte loads per thread
  static_assert(ROWS * RC % NT == 0, "tile must split evenly over the threads");
  uint4 v[kDirect ? 1 : N];

  __device__ __forceinline__ void load(const uint8_t* __restrict__ gsrc, int valid, int tid, uint8_t* lds) {
    load_part<0, N>(gsrc, valid, tid, lds);
  }
  template <int J0, int J1>
  __device__ __forceinline__ void load_part(const uint8_t* __restrict__ gsrc, int valid, int tid, uint8_t* lds) {
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(gsrc), (short)0, valid * RC * 16, kRsrcWord3);
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
#pragma unroll
    for (int j = J0; j < J1; ++j) {
      const int sl = tid + j * NT;
      const int r = sl / RC, pc = sl - (sl / RC) * RC;
      const int off = r * (RC * 16) + 16 * swz<RC>(r, pc);
      if constexpr (kDirect) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rs, (__attribute__((address_space(3))) void*)(lds + 16 * (64 * wv + j * NT)), 16, off, 0, 0, 0);
      } else {
        const u32x4 t = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0);
        v[j] = make_uint4(t[0], t[1], t[2], t[3]);
      }
    }
  }
  __device__ __forceinline__ void commit(uint8_t* lds, int tid) const {
    if constexpr (!kDirect) {
#pragma unroll
      for (int j = 0; j < N; ++j) *reinterpret_cast<uint4*>(lds + 16 * (tid + j * NT)) = v[j];
    }
  }
};

// Wait until at most N of this wave's vector-memory loads are outstanding (s_waitcnt with the
// export and LDS counters left at their maxima, i.e. not waited for).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | (((N >> 4) & 3) << 14));
}

// Workgroup barrier without a memory fence (LDS traffic is ordered by lgkmcnt; global loads that
// are still in flight belong to the next tile and must not be waited for here).
__device__ __forceinline__ void bar() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0), visible to the compiler's own wait tracking
  asm volatile("s_barrier" ::: "memory");
}

template <int B, int D, int PH>
__device__ __forceinline__ const uint8_t* k_tile_src(const Geo& g, const Ws& w, int bh, int kb) {
  const size_t krow0 = (size_t)bh * g.Np + (size_t)kb * B;
  return PH == 0 ? reinterpret_cast<const uint8_t*>(w.k_bf16 + krow0 * D)
       : PH == 3 ? reinterpret_cast<const uint8_t*>(w.k_nv_bf16 + krow0 * D)
       : PH == 1 ? reinterpret_cast<const uint8_t*>(w.k_i8 + krow0 * D)
                 : w.k_fp4 + krow0 * (D / 2);
}

template <int B, int D, int PH>
__device__ __forceinline__ const uint8_t* v_tile_src(const Geo& g, const Ws& w, int bh, int kb) {
  using C = AttnCfg<B, D>;
  return PH == 0
             ? reinterpret_cast<const uint8_t*>(w.vt_bf16 + ((size_t)bh * g.Nb + kb) * (size_t)D * B)
             : w.vt_fp8 + ((size_t)bh * g.Nb + kb) * (size_t)D * C::KP8;
}

// Section clocks (the diagnostic instantiation only): per phase, the shader-clock cycles of the
// key-block loop's parts summed over waves -- 0 wait for K, 1 first barrier, 2 Q K^T and the
// statistics, 3 wait for V, 4 second barrier, 5 P V -- then 6 the wave-blocks counted and, in phase
// 0's row, 7 the summed lifetimes of the waves.
constexpr int kClkPerPhase = 8;
__device__ __forceinline__ unsigned long long clk_now() { return __builtin_amdgcn_s_memtime(); }

// All key blocks of one precision phase (PH = 0: 16-bit, 1: 8-bit, 2: 4-bit) for this row.
// Only this phase's Q operand is live, so the three phases do not compete for registers.
template <int B, int D, int PH, bool kClk>
__device__ __forceinline__ void run_phase(const Geo& g, const Ws& w, const RowCtx& c,
                                          f32x16 (&O)[AttnCfg<B, D>::DT], float& m_run,
                                          float& l_run, int np, int off, uint8_t* sK, uint8_t* sV,
                                          uint8_t* sKs, float* sBias, unsigned long long* clk) {
  using C = AttnCfg<B, D>;
  const int gh = c.gh;
  const float inv_sqrt_d = 1.0f / sqrtf((float)D);

  // Q operand for this phase, straight from the packed workspace
  constexpr bool kQk16 = PH == 0 || PH == 3;  // bf16 Q K^T (16-bit level, NVFP4 4-bit level)
  constexpr int NQ = kQk16 ? D / 16 : (PH == 1 ? D / 32 : D / 64);
  uint4 qop[NQ];
  int qsc[NQ];
  float s_q = 0.0f;
#pragma unroll
  for (int ks = 0; ks < NQ; ++ks) {
    const uint8_t* base =
        PH == 0 ? reinterpret_cast<const uint8_t*>(w.q_bf16 + c.qrow * D) + 32 * ks + 16 * gh
        : PH == 3 ? reinterpret_cast<const uint8_t*>(w.q_nv_bf16 + c.qrow * D) + 32 * ks + 16 * gh
        : PH == 1 ? reinterpret_cast<const uint8_t*>(w.q_i8 + c.qrow * D) + 32 * ks + 16 * gh
                  : w.q_fp4 + c.qrow * (D / 2) + 32 * ks + 16 * gh;
    qop[ks] = c.qok ? *reinterpret_cast<const uint4*>(base) : make_uint4(0, 0, 0, 0);
    qsc[ks] = (PH == 2 && c.qok) ? (int)w.q_e8m0[c.qrow * (D / 32) + 2 * ks + gh] : 127;
  }
  if (PH == 1) s_q = __uint_as_float(uniform_load(reinterpret_cast<const uint32_t*>(w.q_i8_scale) + (size_t)c.bh * g.Nb + c.qb));
  float nv_t = 0.0f;  // NVFP4: product of the Q and K tensor scales of this head
  if (PH == 3) {
    const uint32_t* ts = reinterpret_cast<const uint32_t*>(w.nv_tscale) + (size_t)c.bh * 2;
    nv_t = __uint_as_float(uniform_load(ts)) * __uint_as_float(uniform_load(ts + 1));
  }
  using P = PhaseCfg<B, D, PH>;
  const int lane = c.tid & 63;
  TileMover<C::KT, P::KRC, C::NT, C::DIRECT> kt;
  TileMover<D, P::VRC, C::NT, C::DIRECT> vt;
  uint32_t kscale = 0;  // E8M0 key scales of the staged tile (4-bit phase), 4 bytes per thread

  // The current key block and its INT8 scale (8-bit phase) are carried from one iteration to the
  // next: each iteration loads only the next block's list entry (and scale).
  const float* ks8 = w.k_i8_scale + (size_t)c.bh * g.Nb;
  int kb = list_at(c, off);
  float sk = PH == 1 ? __uint_as_float(uniform_load(reinterpret_cast<const uint32_t*>(ks8) + kb)) : 0.0f;

  // prologue: the first key block's K is loaded
  kt.load(k_tile_src<B, D, PH>(g, w, c.bh, kb), B, c.tid, sK);
  if (PH == 2 && c.tid < C::KT * (D / 32) / 4)
    kscale = c.tid < B * (D / 32) / 4
                 ? *reinterpret_cast<const uint32_t*>(w.k_e8m0 + ((size_t)c.bh * g.Np + (size_t)kb * B) * (D / 32) + 4 * c.tid)
                 : 0x7f7f7f7fu;

  unsigned long long ck[6] = {0, 0, 0, 0, 0, 0}, t_prev = 0;
  auto tick = [&](int part) {  // adds the cycles since the previous tick to part
    if constexpr (kClk) {
      const unsigned long long t = clk_now();
      if (part >= 0) ck[part] += t - t_prev;
      t_prev = t;
    }
  };
  for (int it = 0; it < np; ++it) {
    tick(-1);
    // consumed at the end of this iteration (its latency hides behind the barrier and Q K^T)
    const int kb_next = list_at(c, off + min(it + 1, np - 1));  // the last block re-reads its own entry
    const float sk_next = PH == 1 ? __uint_as_float(uniform_load(reinterpret_cast<const uint32_t*>(ks8) + kb_next)) : 0.0f;
    // real extent of key block kb (regions at the high-y / high-x edge hold padding)
    const int per = g.nby * g.nbx;
    const int rem = kb % per;
    const int ry = rem / g.nbx, rx = rem - ry * g.nbx;
    const int vh = min(g.rh, g.H - ry * g.rh), vw = min(g.rw, g.W - rx * g.rw);
    const bool full = vh == g.rh && vw == g.rw && B == C::KT;
    // Two barriers per key block.  sK, sKs and sBias were last read by the previous Q K^T, which
    // every wave finished before the barrier ahead of the previous P V, so they are written here
    // without a barrier of their own; sV is free once every wave reaches the barrier below.
    kt.commit(sK, c.tid);
    if constexpr (!C::DIRECT) vt.load(v_tile_src<B, D, PH>(g, w, c.bh, kb), D, c.tid, sV);
    if (PH == 2 && c.tid < C::KT * (D / 32) / 4) *reinterpret_cast<uint32_t*>(sKs + 4 * c.tid) = kscale;
    if (!full && c.tid < C::KT) {
      const int m = c.tid, iy = m / g.rw, ix = m - (m / g.rw) * g.rw;
      sBias[m] = (m < B && iy < vh && ix < vw) ? 0.0f : -INFINITY;
    }
    if constexpr (C::DIRECT) wait_vm<0>();  // K (issued one key block earlier) has landed
    tick(0);
    bar();  // K, scales and bias visible; every wave is done with the previous P V
    tick(1);
    // This tile's V streams in while Q K^T and the softmax run; its loads are issued a quarter after
    // each m-tile's products, so the first products do not wait behind the whole tile's issue.
    constexpr int NVL = TileMover<D, P::VRC, C::NT, C::DIRECT>::N;
    static_assert(!C::DIRECT || C::MT == 4, "direct loads: 128-token blocks");  // quarters may be empty
    const uint8_t* vsrc = v_tile_src<B, D, PH>(g, w, c.bh, kb);
    auto v_part = [&](int mt) {  // mt is a constant in the unrolled loop below
      if constexpr (C::DIRECT) {
        if (mt == 0) vt.template load_part<0, NVL / 4>(vsrc, D, c.tid, sV);
        if (mt == 1) vt.template load_part<NVL / 4, NVL / 2>(vsrc, D, c.tid, sV);
        if (mt == 2) vt.template load_part<NVL / 2, 3 * NVL / 4>(vsrc, D, c.tid, sV);
        if (mt == 3) vt.template load_part<3 * NVL / 4, NVL>(vsrc, D, c.tid, sV);
      }
    };
    // per-lane LDS addresses are recomputed in every iteration (a few integer ops) instead of
    // being hoisted out of the loop, where they would pin dozens of registers
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int nl = ln & 31, gl = ln >> 5;
    // Logical chunk 2j + gl of operand row nl sits at byte nl*RB + 16*((2j + gl) ^ sw), sw the
    // row's swizzle; 2j and gl occupy disjoint bits, so that is (nl*RB + 16*(gl ^ sw)) ^ (32 j):
    // one per-lane base per tile and one XOR per 16-byte read.
    const int kbase = nl * P::KRB + 16 * (gl ^ ((nl / (16 / P::KRC)) % P::KRC));

    // ---- S^T = K Q^T; each finished m-tile's raw maximum is folded in while the next m-tile's
    // products run (full blocks: the scale is applied to the maximum once, c_scale > 0 keeps the
    // order and c_scale = 0 gives 0 either way)
    float c_scale = kLog2e * inv_sqrt_d;
    if (PH == 1)
      c_scale = s_q * sk *
                (kLog2e * inv_sqrt_d);
    if (PH == 3)  // NVFP4: the operands carry the group scales, the tensor scales apply here
      c_scale = nv_t * (kLog2e * inv_sqrt_d);
    f32x16 S[C::MT];  // the 8-bit phase keeps its int32 sums here (bit patterns) until converted
    float mx = -INFINITY;
    auto qk_tile = [&](int mt) {
      if (kQk16) {
        f32x16 acc = {};
#pragma unroll
        for (int ks = 0; ks < NQ; ++ks)
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_bit_cast(bf16x8, lds16(sK + 32 * mt * P::KRB + (kbase ^ (32 * ks)))),
              __builtin_bit_cast(bf16x8, qop[ks]), acc, 0, 0, 0);
        S[mt] = acc;
      } else if (PH == 1) {
        i32x16 acc = {};
#pragma unroll
        for (int ks = 0; ks < NQ; ++ks)
          acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(
              __builtin_bit_cast(i32x4, lds16(sK + 32 * mt * P::KRB + (kbase ^ (32 * ks)))),
              __builtin_bit_cast(i32x4, qop[ks]), acc, 0, 0, 0);
        S[mt] = __builtin_bit_cast(f32x16, acc);
      } else {
        f32x16 acc = {};
#pragma unroll
        for (int ks = 0; ks < NQ; ++ks) {
          const uint4 u = lds16(sK + 32 * mt * P::KRB + (kbase ^ (32 * ks)));
          const i32x8 a = {(int)u.x, (int)u.y, (int)u.z, (int)u.w, 0, 0, 0, 0};
          const i32x8 b = {(int)qop[ks].x, (int)qop[ks].y, (int)qop[ks].z, (int)qop[ks].w, 0, 0, 0, 0};
          const int ksc = (int)sKs[(32 * mt + nl) * (D / 32) + 2 * ks + gl];
          acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc, 4, 4, 0, ksc, 0, qsc[ks]);
        }
        S[mt] = acc;
      }
    };
    // kFull: the block has no padding keys, known at compile time (low-bit phases) or at run
    // time (16-bit phase)
    auto qk_post = [&](int mt, auto full_c) {
      constexpr bool kFull = decltype(full_c)::value;
      if (PH == 1) {
        const i32x16 si = __builtin_bit_cast(i32x16, S[mt]);
#pragma unroll
        for (int r = 0; r < 16; ++r) S[mt][r] = (float)si[r];
      }
      if (kFull || (kQk16 && full)) {
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, S[mt][r]);
      } else {
        // edge block: scale, then pad keys (and key slots beyond B) get -inf from sBias
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const float4 bias4 = *reinterpret_cast<const float4*>(sBias + 32 * mt + 8 * r4 + 4 * gl);
          S[mt][4 * r4 + 0] = S[mt][4 * r4 + 0] * c_scale + bias4.x;
          S[mt][4 * r4 + 1] = S[mt][4 * r4 + 1] * c_scale + bias4.y;
          S[mt][4 * r4 + 2] = S[mt][4 * r4 + 2] * c_scale + bias4.z;
          S[mt][4 * r4 + 3] = S[mt][4 * r4 + 3] * c_scale + bias4.w;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, S[mt][r]);
      }
    };
    // one m-tile of lookahead: the products of m-tile mt are issued before m-tile mt - 1's
    // conversion and maximum, which then run while the matrix core works
    auto qk_all = [&](auto full_c) {
      qk_tile(0);
      v_part(0);
#pragma unroll
      for (int mt = 1; mt < C::MT; ++mt) {
        qk_tile(mt);
        v_part(mt);
        qk_post(mt - 1, full_c);
      }
      qk_post(C::MT - 1, full_c);
    };
    // Low-bit phases take the full / edge choice once per key block, so each copy of the pipeline
    // is straight-line code in which the scheduler can interleave products, conversions and
    // maxima.  The 16-bit phase keeps the choice per m-tile: two copies of it do not fit in the
    // registers.
    if (!kQk16 && full)
      qk_all(std::true_type{});
    else
      qk_all(std::false_type{});

    // ---- online softmax statistics in the log2 domain, one running-max update per key block
    mx = halves_max(mx);
    if (full) mx *= c_scale;
    const float m_new = fmaxf(m_run, mx);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    const float nbias = PH == 0 ? -m_new : 8.0f - m_new;  // low-bit phases produce 2^8 P
    const float cs = full ? c_scale : 1.0f;
    m_run = m_new;
    if (!__all(alpha == 1.0f)) {
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) O[dt][r] *= alpha;
    }

    // ---- O^T += V^T P^T.  Once V is in LDS and every wave is past its Q K^T, the next key
    // block's K streams in during the products.  P is produced chunk by chunk right before the
    // products that consume it, so its exponentials can run under the previous chunk's
    // matrix-core work.
    tick(2);
    if constexpr (C::DIRECT) wait_vm<0>();
    vt.commit(sV, c.tid);
    tick(3);
    bar();  // V visible; every wave is done with sK
    tick(4);
    // The P V section carries most of the VALU work; the other wave on the SIMD is then usually in
    // its Q K^T, which needs the matrix core far more than the VALU.  Raising this wave's issue
    // priority while its exponentials run lets both proceed (16- and 8-bit phases: -0.5 to -1.5 %
    // on the 720p maps, bit-identical; at 4 bit it was slower).
    if constexpr (PH <= 1) __builtin_amdgcn_s_setprio(1);
    if (it + 1 < np) kt.load(k_tile_src<B, D, PH>(g, w, c.bh, kb_next), B, c.tid, sK);
    if (PH == 2 && c.tid < C::KT * (D / 32) / 4)
      kscale = c.tid < B * (D / 32) / 4
                   ? *reinterpret_cast<const uint32_t*>(w.k_e8m0 + ((size_t)c.bh * g.Np + (size_t)kb_next * B) * (D / 32) + 4 * c.tid)
                   : 0x7f7f7f7fu;
    // V^T rows: 16-bit tiles read chunks 2 c16 + gl, low-bit tiles chunks 4 c64 + 2 gl + h (h = 0, 1);
    // the same disjoint-bit argument gives one base per lane and XORs
    const int vsw = (nl / (16 / P::VRC)) % P::VRC;
    const int vbase = nl * P::VRB + 16 * (PH == 0 ? (gl ^ vsw) : ((2 * gl) ^ vsw));
    float psum = 0.0f;
    if (PH == 0) {
#pragma unroll
      for (int c16 = 0; c16 < B / 16; ++c16) {
        const int mt = c16 >> 1, rb = 8 * (c16 & 1);
        float p[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          p[j] = __builtin_amdgcn_exp2f(fmaf(S[mt][rb + j], cs, nbias));
          psum += p[j];
        }
        const bf16x8 bop = __builtin_bit_cast(
            bf16x8, make_uint4(pack_bf16(p[0], p[1]), pack_bf16(p[2], p[3]), pack_bf16(p[4], p[5]),
                               pack_bf16(p[6], p[7])));
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt) {
          const bf16x8 a =
              __builtin_bit_cast(bf16x8, lds16(sV + 32 * dt * P::VRB + (vbase ^ (32 * c16))));
          O[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bop, O[dt], 0, 0, 0);
        }
      }
    } else {
#pragma unroll
      for (int c64 = 0; c64 < C::KP8 / 64; ++c64) {
        i32x8 bop;
#pragma unroll
        for (int hsel = 0; hsel < 2; ++hsel) {
          const int mt = 2 * c64 + hsel;
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            int word = 0;
            if (mt < C::MT) {
              float p[4];
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                p[e] = __builtin_amdgcn_exp2f(fmaf(S[mt < C::MT ? mt : 0][4 * q4 + e], cs, nbias));
                psum += p[e];
              }
              // the old-value operand is any register: both halves are written
              word = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], __float_as_int(p[0]), false);
              word = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], word, true);
            }
            bop[4 * hsel + q4] = word;
          }
        }
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt) {
          const uint8_t* vp = sV + 32 * dt * P::VRB;
          const int va = vbase ^ (64 * c64);
          const uint4 u0 = lds16(vp + va);
          const uint4 u1 = lds16(vp + (va ^ 16));
          const i32x8 a = {(int)u0.x, (int)u0.y, (int)u0.z, (int)u0.w,
                           (int)u1.x, (int)u1.y, (int)u1.z, (int)u1.w};
          O[dt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, bop, O[dt], 0, 0, 0, kScaleOne,
                                                                  0, kScaleOne);
        }
      }
      psum *= 0.00390625f;  // 2^-8, exact
    }
    if constexpr (PH <= 1) __builtin_amdgcn_s_setprio(0);
    l_run = alpha * l_run + psum;
    kb = kb_next;
    sk = sk_next;
    tick(5);
  }
  if constexpr (kClk) {
    if ((c.tid & 63) == 0) {
#pragma unroll
      for (int i = 0; i < 6; ++i) atomicAdd(clk + PH * kClkPerPhase + i, ck[i]);
      atomicAdd(clk + PH * kClkPerPhase + 6, (unsigned long long)np);
    }
  }
}

// kNv: the 4-bit level runs in NVFP4 (phase 3) instead of MXFP4 (phase 2); a separate
// instantiation, so that each kernel holds the registers of its own phases only
// kClk: the section-clock diagnostic (clk holds 4 x kClkPerPhase counters); off, the kernel
// reads no clock and clk is unused
template <int B, int D, bool kNv, bool kClk>
__global__ __launch_bounds__(64 * (B >= 32 ? B / 32 : 1)) __attribute__((amdgpu_waves_per_eu(2)))
void attn_kernel(Geo g, Ws w, unsigned long long* clk) {
  using C = AttnCfg<B, D>;
  __shared__ __attribute__((aligned(16))) uint8_t sK[C::KBYTES];
  __shared__ __attribute__((aligned(16))) uint8_t sV[C::VBYTES];
  __shared__ __attribute__((aligned(16))) uint8_t sKs[C::SBYTES];
  __shared__ __attribute__((aligned(16))) float sBias[C::KT];

  // Workgroups are dispatched round-robin over the 8 dies: workgroup id x + 8j runs on die x and
  // takes entry j of that die's slice of the work order.
  unsigned long long t_start = 0;
  if constexpr (kClk) t_start = clk_now();
  RowCtx c;
  const int Nb = g.Nb;
  if (!stage_ok(uniform_load(w.stage), uniform_load(w.stage + 1), g.tag,
                stage_bit(DAP_STAGE_RANKED) | stage_bit(DAP_STAGE_ATTENDED))) {
    // the ranking has not run on this workspace for this configuration: the order, counts and
    // lists are not to be trusted, so workgroup i writes zeros over row i of the packed output
    const long long i = blockIdx.x;
    if (i >= (long long)g.bh * Nb) return;
    uint4* dst = reinterpret_cast<uint4*>(w.out + (size_t)i * B * D);  // row i = bh * Nb + qb
    for (int t = threadIdx.x; t < B * D / 8; t += C::NT) dst[t] = make_uint4(0, 0, 0, 0);
    return;
  }
  {
    const int x = blockIdx.x & (kXcds - 1), j = blockIdx.x / kXcds;
    if (j >= g.bh * xcd_chunk_size(x, Nb)) return;
    const uint32_t item = w.order[(size_t)x * xcd_stride(g.bh, Nb) + j];
    c.bh = __builtin_amdgcn_readfirstlane((int)(item >> 16));
    c.qb = __builtin_amdgcn_readfirstlane((int)(item & 0xffff));
    if (c.bh >= g.bh || c.qb >= Nb) return;  // cannot happen for an order the ranking wrote
  }
  c.tid = threadIdx.x;
  const int wv = c.tid >> 6, lane = c.tid & 63;
  c.n = lane & 31;
  c.gh = lane >> 5;
  const int qr = 32 * wv + c.n;  // query row inside the block
  c.qok = qr < B;
  c.qrow = (size_t)c.bh * g.Np + (size_t)c.qb * B + qr;
  c.lists = reinterpret_cast<const uint32_t*>(w.lists);
  c.lbase = (size_t)c.bh * g.pairs + (size_t)c.qb * Nb;
  c.nb_last = Nb - 1;

  const int32_t* cnt = w.counts + ((size_t)c.bh * Nb + c.qb) * 4;
  // counts clamped so that no list is walked past its row (a no-op for counts the ranking wrote)
  const int n16 = min(max((int)uniform_load(reinterpret_cast<const uint32_t*>(cnt)), 0), Nb);
  const int n8 = min(max((int)uniform_load(reinterpret_cast<const uint32_t*>(cnt) + 1), 0), Nb - n16);
  const int n4 = min(max((int)uniform_load(reinterpret_cast<const uint32_t*>(cnt) + 2), 0), Nb - n16 - n8);

  f32x16 O[C::DT];
#pragma unroll
  for (int i = 0; i < C::DT; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) O[i][r] = 0.0f;
  float m_run = -INFINITY, l_run = 0.0f;

  if (n16 > 0) run_phase<B, D, 0, kClk>(g, w, c, O, m_run, l_run, n16, 0, sK, sV, sKs, sBias, clk);
  const bool lowbit = n8 + n4 > 0;
  // The FP8 V scales of this lane's accumulator channels 32 dt + 8 r4 + 4 gh + e: four
  // consecutive channels per (dt, r4), fetched together as 16-byte loads.
  auto v_scales = [&](float4 (&sv)[C::DT][4]) {
    const float* vs = w.v_scale + (size_t)c.bh * D + 4 * c.gh;
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) sv[dt][r4] = *reinterpret_cast<const float4*>(vs + 32 * dt + 8 * r4);
  };
  if (lowbit) {
    // accumulator unit change at the 16 -> low-bit boundary: channel d x 2^8 / s_V[d]
    float4 sv[C::DT][4];
    v_scales(sv);
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const float s4[4] = {sv[dt][r4].x, sv[dt][r4].y, sv[dt][r4].z, sv[dt][r4].w};
#pragma unroll
        // (O 2^8) / s rather than O (2^8 / s): the quotient stays finite for the tiniest
        // nonzero scales, whose reciprocal would overflow
        for (int e = 0; e < 4; ++e) O[dt][4 * r4 + e] = s4[e] > 0.0f ? (O[dt][4 * r4 + e] * 256.0f) / s4[e] : 0.0f;
      }
  }
  if (n8 > 0) run_phase<B, D, 1, kClk>(g, w, c, O, m_run, l_run, n8, n16, sK, sV, sKs, sBias, clk);
  if (n4 > 0) run_phase<B, D, kNv ? 3 : 2, kClk>(g, w, c, O, m_run, l_run, n4, n16 + n8, sK, sV, sKs, sBias, clk);

  // ---- finalise: O / l (0 when no pair was kept), undo the low-bit units, bf16 out
  const float l = halves_sum(l_run);
  const float inv_l = l > 0.0f ? 1.0f / l : 0.0f;
  if (c.qok) {
    uint16_t* dst = w.out + c.qrow * D;
    float4 sv[C::DT][4];
    if (lowbit) v_scales(sv);
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d0 = 32 * dt + 8 * r4 + 4 * c.gh;
        const float s4[4] = {sv[dt][r4].x, sv[dt][r4].y, sv[dt][r4].z, sv[dt][r4].w};
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float o = O[dt][4 * r4 + e];
          if (lowbit) o *= s4[e] * 0.00390625f;
          v[e] = o * inv_l;
        }
        const __bf16 b0 = (__bf16)v[0], b1 = (__bf16)v[1], b2 = (__bf16)v[2], b3 = (__bf16)v[3];
        const uint32_t lo = (uint32_t)__builtin_bit_cast(uint16_t, b0) |
                            ((uint32_t)__builtin_bit_cast(uint16_t, b1) << 16);
        const uint32_t hi = (uint32_t)__builtin_bit_cast(uint16_t, b2) |
                            ((uint32_t)__builtin_bit_cast(uint16_t, b3) << 16);
        *reinterpret_cast<uint2*>(dst + d0) = make_uint2(lo, hi);
      }
  }
  if constexpr (kClk) {
    if ((c.tid & 63) == 0) atomicAdd(clk + 7, clk_now() - t_start);
  }
}

template <int B, int D, bool kClk>
hipError_t attn_bd(const Geo& g, const Ws& w, unsigned long long* clk, hipStream_t s) {
  using C = AttnCfg<B, D>;
  const unsigned grid = (unsigned)(kXcds * xcd_stride(g.bh, g.Nb));
  if (g.fp4_format == DAP_FP4_NVFP4)
    attn_kernel<B, D, true, kClk><<<grid, C::NT, 0, s>>>(g, w, clk);
  else
    attn_kernel<B, D, false, kClk><<<grid, C::NT, 0, s>>>(g, w, clk);
  return hipGetLastError();
}

template <bool kClk>
hipError_t attn_any(const Geo& g, const Ws& w, unsigned long long* clk, hipStream_t s) {
  if (g.D == 64) {
    if (g.B == 16) return attn_bd<16, 64, kClk>(g, w, clk, s);
    if (g.B == 64) return attn_bd<64, 64, kClk>(g, w, clk, s);
    return attn_bd<128, 64, kClk>(g, w, clk, s);
  }
  if (g.B == 16) return attn_bd<16, 128, kClk>(g, w, clk, s);
  if (g.B == 64) return attn_bd<64, 128, kClk>(g, w, clk, s);
  return attn_bd<128, 128, kClk>(g, w, clk, s);
}

}  // namespace

hipError_t launch_attention(const Geo& g, const Ws& w, hipStream_t s) {
  return attn_any<false>(g, w, nullptr, s);
}

hipError_t launch_attention_clocked(const Geo& g, const Ws& w, unsigned long long* clk, hipStream_t s) {
  return attn_any<true>(g, w, clk, s);
}

}  // namespace dap
