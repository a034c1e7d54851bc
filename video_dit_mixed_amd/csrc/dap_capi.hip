// libdap C ABI: argument validation, workspace layout and the four stream-ordered calls.
// Validation is pure host code and runs before any HIP call.
#include <math.h>
#include <string.h>

#include "dap_internal.h"

namespace {

using dap::Geo;
using dap::Ws;

constexpr uint64_t kAlign = 256;
inline uint64_t align_up(uint64_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

dap_status validate(const dap_config* c) {
  if (!c) return DAP_E_INVALID;
  if (c->batch < 1 || c->heads < 1 || c->T < 1 || c->H < 1 || c->W < 1 || c->region_h < 1 ||
      c->region_w < 1)
    return DAP_E_INVALID;
  if (!(c->lambda >= 0.0 && c->lambda <= 1.0)) return DAP_E_INVALID;  // also rejects NaN
  long long qsum = 0;
  for (int i = 0; i < 4; ++i) {
    if (c->quota_bp[i] < 0) return DAP_E_INVALID;
    qsum += c->quota_bp[i];
  }
  if (qsum > 10000) return DAP_E_INVALID;
  if (c->fp4_format != DAP_FP4_MXFP4 && c->fp4_format != DAP_FP4_NVFP4) return DAP_E_INVALID;
  if (c->head_dim != 64 && c->head_dim != 128) return DAP_E_UNSUPPORTED;
  const long long B = (long long)c->region_h * c->region_w;
  if (B != 16 && B != 64 && B != 128) return DAP_E_UNSUPPORTED;
  // widened before any arithmetic, and each factor bounded before the product, so that no
  // configuration overflows on its way to the check
  const long long nby = ((long long)c->H + c->region_h - 1) / c->region_h;
  const long long nbx = ((long long)c->W + c->region_w - 1) / c->region_w;
  if (c->T > 4096 || nby > 4096 || nbx > 4096) return DAP_E_UNSUPPORTED;
  const long long Nb = (long long)c->T * nby * nbx;
  if (Nb > 4096) return DAP_E_UNSUPPORTED;  // pair index must fit 24 bits; lists are uint16
  const long long bh = (long long)c->batch * c->heads;
  if (bh > 65535) return DAP_E_UNSUPPORTED;
  return DAP_OK;
}

// FNV-1a over every field of the configuration: the tag a workspace's stage word carries, so that
// a stage left by a layer of another shape or quota is not taken for this one's.
uint32_t config_tag(const dap_config* c) {
  uint32_t h = 2166136261u;
  auto mix = [&](const void* p, size_t n) {
    const unsigned char* b = static_cast<const unsigned char*>(p);
    for (size_t i = 0; i < n; ++i) h = (h ^ b[i]) * 16777619u;
  };
  const int32_t ints[] = {c->batch, c->heads, c->head_dim, c->T, c->H, c->W, c->region_h,
                          c->region_w, c->quota_bp[0], c->quota_bp[1], c->quota_bp[2],
                          c->quota_bp[3], c->fp4_format};
  mix(ints, sizeof(ints));
  mix(&c->lambda, sizeof(c->lambda));
  return h;
}

void make_geo(const dap_config* c, Geo* g) {
  memset(g, 0, sizeof(*g));
  g->bh = c->batch * c->heads;
  g->heads = c->heads;
  g->D = c->head_dim;
  g->T = c->T;
  g->H = c->H;
  g->W = c->W;
  g->rh = c->region_h;
  g->rw = c->region_w;
  g->nby = (c->H + c->region_h - 1) / c->region_h;
  g->nbx = (c->W + c->region_w - 1) / c->region_w;
  g->Hp = g->nby * g->rh;
  g->Wp = g->nbx * g->rw;
  g->Nb = c->T * g->nby * g->nbx;
  g->B = g->rh * g->rw;
  g->Np = g->Nb * g->B;
  g->kp8 = (g->B + 63) / 64 * 64;
  g->N = c->T * c->H * c->W;
  g->pairs = (long long)g->Nb * g->Nb;
  const long long q4 = c->quota_bp[1], q8 = c->quota_bp[2], q16 = c->quota_bp[3];
  auto rnd = [&](long long x) { return (g->pairs * x + 5000) / 10000; };
  g->c16 = rnd(q16);
  g->c8 = rnd(q16 + q8);
  g->c4 = rnd(q16 + q8 + q4);
  g->lambda = c->lambda;
  g->need16 = g->c16 > 0;
  g->need8 = g->c8 > g->c16;
  g->need4 = g->c4 > g->c8;
  g->fp4_format = c->fp4_format;
  g->tag = config_tag(c);
}

void make_layout(const Geo& g, dap_layout* L) {
  memset(L, 0, sizeof(*L));
  L->Hp = g.Hp;
  L->Wp = g.Wp;
  L->nby = g.nby;
  L->nbx = g.nbx;
  L->Nb = g.Nb;
  L->B = g.B;
  L->Np = g.Np;
  L->kp8 = g.kp8;
  L->bh = g.bh;
  L->D = g.D;
  L->pairs = g.pairs;
  L->c16 = g.c16;
  L->c8 = g.c8;
  L->c4 = g.c4;
  const uint64_t bh = g.bh, Np = g.Np, Nb = g.Nb, D = g.D;
  uint64_t o = 0;
  auto take = [&](uint64_t bytes) {
    uint64_t at = o;
    o = align_up(o + bytes);
    return at;
  };
  L->off_q_bf16 = take(bh * Np * D * 2);
  L->off_k_bf16 = take(bh * Np * D * 2);
  L->off_vt_bf16 = take(bh * Np * D * 2);
  L->off_q_i8 = take(bh * Np * D);
  L->off_k_i8 = take(bh * Np * D);
  L->off_q_i8_scale = take(bh * Nb * 4);
  L->off_k_i8_scale = take(bh * Nb * 4);
  L->off_q_fp4 = take(bh * Np * D / 2);
  L->off_k_fp4 = take(bh * Np * D / 2);
  L->off_q_e8m0 = take(bh * Np * D / 32);
  L->off_k_e8m0 = take(bh * Np * D / 32);
  L->off_vt_fp8 = take(bh * Nb * D * (uint64_t)g.kp8);
  L->off_v_scale = take(bh * D * 4);
  L->off_v_amax = take(bh * D * 4);
  L->off_q_avg = take(bh * Nb * D * 8);
  L->off_q_max = take(bh * Nb * D * 8);
  L->off_k_avg = take(bh * Nb * D * 8);
  L->off_k_max = take(bh * Nb * D * 8);
  L->off_scores = take(bh * Nb * Nb * 8);
  L->off_lmax = take(bh * Nb * Nb * 8);
  L->off_rank_state = take(bh * 3 * sizeof(dap::RankCut));
  L->off_rank_hist = take(bh * 3 * dap::kRankBins * 4);
  L->off_map = take(bh * Nb * Nb);
  L->off_lists = take(bh * Nb * Nb * 2);
  L->off_counts = take(bh * Nb * 4 * 4);
  L->off_out = take(bh * Np * D * 2);
  L->off_zeros = take(256);
  L->off_order = take((uint64_t)dap::kXcds * dap::xcd_stride(g.bh, g.Nb) * 4);
  L->off_stage = take(8);
  const uint64_t nv = g.fp4_format == DAP_FP4_NVFP4 ? 1 : 0;  // NVFP4 sections, empty otherwise
  L->off_q_nv_scale = take(nv * bh * Np * D / 16);
  L->off_k_nv_scale = take(nv * bh * Np * D / 16);
  L->off_q_nv_bf16 = take(nv * bh * Np * D * 2);
  L->off_k_nv_bf16 = take(nv * bh * Np * D * 2);
  L->off_nv_tscale = take(nv * bh * 2 * 4);
  L->off_qk_amax = take(nv * 2 * bh * D * 4);
  L->total_bytes = o;
}

Ws make_ws(void* base, const dap_layout& L) {
  char* b = static_cast<char*>(base);
  Ws w;
  w.q_bf16 = reinterpret_cast<uint16_t*>(b + L.off_q_bf16);
  w.k_bf16 = reinterpret_cast<uint16_t*>(b + L.off_k_bf16);
  w.vt_bf16 = reinterpret_cast<uint16_t*>(b + L.off_vt_bf16);
  w.q_i8 = reinterpret_cast<int8_t*>(b + L.off_q_i8);
  w.k_i8 = reinterpret_cast<int8_t*>(b + L.off_k_i8);
  w.q_i8_scale = reinterpret_cast<float*>(b + L.off_q_i8_scale);
  w.k_i8_scale = reinterpret_cast<float*>(b + L.off_k_i8_scale);
  w.q_fp4 = reinterpret_cast<uint8_t*>(b + L.off_q_fp4);
  w.k_fp4 = reinterpret_cast<uint8_t*>(b + L.off_k_fp4);
  w.q_e8m0 = reinterpret_cast<uint8_t*>(b + L.off_q_e8m0);
  w.k_e8m0 = reinterpret_cast<uint8_t*>(b + L.off_k_e8m0);
  w.vt_fp8 = reinterpret_cast<uint8_t*>(b + L.off_vt_fp8);
  w.v_scale = reinterpret_cast<float*>(b + L.off_v_scale);
  w.v_amax = reinterpret_cast<uint32_t*>(b + L.off_v_amax);
  w.q_avg = reinterpret_cast<double*>(b + L.off_q_avg);
  w.q_max = reinterpret_cast<double*>(b + L.off_q_max);
  w.k_avg = reinterpret_cast<double*>(b + L.off_k_avg);
  w.k_max = reinterpret_cast<double*>(b + L.off_k_max);
  w.scores = reinterpret_cast<double*>(b + L.off_scores);
  w.lmax = reinterpret_cast<double*>(b + L.off_lmax);
  w.rank_state = b + L.off_rank_state;
  w.rank_hist = reinterpret_cast<uint32_t*>(b + L.off_rank_hist);
  w.map = reinterpret_cast<uint8_t*>(b + L.off_map);
  w.lists = reinterpret_cast<uint16_t*>(b + L.off_lists);
  w.counts = reinterpret_cast<int32_t*>(b + L.off_counts);
  w.out = reinterpret_cast<uint16_t*>(b + L.off_out);
  w.zeros = reinterpret_cast<uint8_t*>(b + L.off_zeros);
  w.order = reinterpret_cast<uint32_t*>(b + L.off_order);
  w.stage = reinterpret_cast<uint32_t*>(b + L.off_stage);
  w.q_nv_scale = reinterpret_cast<uint8_t*>(b + L.off_q_nv_scale);
  w.k_nv_scale = reinterpret_cast<uint8_t*>(b + L.off_k_nv_scale);
  w.q_nv_bf16 = reinterpret_cast<uint16_t*>(b + L.off_q_nv_bf16);
  w.k_nv_bf16 = reinterpret_cast<uint16_t*>(b + L.off_k_nv_bf16);
  w.nv_tscale = reinterpret_cast<float*>(b + L.off_nv_tscale);
  w.qk_amax = reinterpret_cast<uint32_t*>(b + L.off_qk_amax);
  return w;
}

inline bool aligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) % kAlign) == 0; }

// Common checks of the four stream calls: config, workspace pointer and size.
dap_status check_call(const dap_config* c, const void* ws, size_t ws_bytes, Geo* g,
                      dap_layout* L) {
  dap_status st = validate(c);
  if (st != DAP_OK) return st;
  if (!ws || !aligned(ws)) return DAP_E_INVALID;
  make_geo(c, g);
  make_layout(*g, L);
  if (ws_bytes < L->total_bytes) return DAP_E_WORKSPACE;
  return DAP_OK;
}

inline dap_status hip_status(hipError_t e) { return e == hipSuccess ? DAP_OK : DAP_E_HIP; }

}  // namespace

extern "C" {

size_t dap_abi_version(void) { return DAP_ABI_VERSION; }

dap_status dap_workspace_bytes(const dap_config* cfg, size_t* bytes) {
  if (!bytes) return DAP_E_INVALID;
  dap_status st = validate(cfg);
  if (st != DAP_OK) return st;
  Geo g;
  dap_layout L;
  make_geo(cfg, &g);
  make_layout(g, &L);
  *bytes = L.total_bytes;
  return DAP_OK;
}

dap_status dap_workspace_layout(const dap_config* cfg, dap_layout* out) {
  if (!out) return DAP_E_INVALID;
  dap_status st = validate(cfg);
  if (st != DAP_OK) return st;
  Geo g;
  make_geo(cfg, &g);
  make_layout(g, out);
  return DAP_OK;
}

dap_status dap_prepare(const dap_config* cfg, const void* q, const void* k, const void* v,
                       void* ws, size_t ws_bytes, hipStream_t stream) {
  Geo g;
  dap_layout L;
  dap_status st = check_call(cfg, ws, ws_bytes, &g, &L);
  if (st != DAP_OK) return st;
  if (!q || !k || !v || !aligned(q) || !aligned(k) || !aligned(v)) return DAP_E_INVALID;
  const Ws w = make_ws(ws, L);
  hipError_t e = dap::launch_prepare(g, static_cast<const uint16_t*>(q),
                                     static_cast<const uint16_t*>(k),
                                     static_cast<const uint16_t*>(v), w, stream);
  if (e == hipSuccess) e = dap::launch_stage(g, w, dap::kStageAny, DAP_STAGE_PREPARED, stream);
  return hip_status(e);
}

dap_status dap_prepare_static_scratch(const dap_config* cfg, const void* q, const void* k,
                                      const void* v, void* ws, size_t ws_bytes,
                                      hipStream_t stream) {
  Geo g;
  dap_layout L;
  dap_status st = check_call(cfg, ws, ws_bytes, &g, &L);
  if (st != DAP_OK) return st;
  if (!q || !k || !v || !aligned(q) || !aligned(k) || !aligned(v)) return DAP_E_INVALID;
  if ((size_t)g.bh * g.D > dap::kStaticScratchWords) return DAP_E_SCRATCH_LIMIT;
  const Ws w = make_ws(ws, L);
  hipError_t e = dap::launch_prepare_static_scratch(g, static_cast<const uint16_t*>(q),
                                                    static_cast<const uint16_t*>(k),
                                                    static_cast<const uint16_t*>(v), w, stream);
  if (e == hipSuccess) e = dap::launch_stage(g, w, dap::kStageAny, DAP_STAGE_PREPARED, stream);
  return hip_status(e);
}

dap_status dap_draft_rank(const dap_config* cfg, void* ws, size_t ws_bytes, uint8_t* map_out,
                          double* scores_out, hipStream_t stream) {
  Geo g;
  dap_layout L;
  dap_status st = check_call(cfg, ws, ws_bytes, &g, &L);
  if (st != DAP_OK) return st;
  if ((map_out && !aligned(map_out)) || (scores_out && !aligned(scores_out)))
    return DAP_E_INVALID;
  Ws w = make_ws(ws, L);
  hipError_t e = dap::launch_draft(g, w, stream);
  if (e == hipSuccess && scores_out)
    e = hipMemcpyAsync(scores_out, w.scores, (size_t)g.bh * g.pairs * 8, hipMemcpyDeviceToDevice,
                       stream);
  if (e == hipSuccess) e = dap::launch_rank(g, w, stream);
  if (e == hipSuccess && map_out)
    e = hipMemcpyAsync(map_out, w.map, (size_t)g.bh * g.pairs, hipMemcpyDeviceToDevice, stream);
  if (e == hipSuccess)
    e = dap::launch_stage(g, w, dap::kAcceptDraftRank, DAP_STAGE_RANKED, stream);
  return hip_status(e);
}

dap_status dap_attention(const dap_config* cfg, void* ws, size_t ws_bytes, hipStream_t stream) {
  Geo g;
  dap_layout L;
  dap_status st = check_call(cfg, ws, ws_bytes, &g, &L);
  if (st != DAP_OK) return st;
  const Ws w = make_ws(ws, L);
  hipError_t e = dap::launch_attention(g, w, stream);
  if (e == hipSuccess)
    e = dap::launch_stage(g, w, dap::kAcceptAttention, DAP_STAGE_ATTENDED, stream);
  return hip_status(e);
}

dap_status dap_attention_section_clocks(const dap_config* cfg, void* ws, size_t ws_bytes,
                                        uint64_t* clocks, hipStream_t stream) {
  Geo g;
  dap_layout L;
  dap_status st = check_call(cfg, ws, ws_bytes, &g, &L);
  if (st != DAP_OK) return st;
  if (!clocks || (reinterpret_cast<uintptr_t>(clocks) & 7) != 0) return DAP_E_INVALID;
  const Ws w = make_ws(ws, L);
  hipError_t e = dap::launch_attention_clocked(g, w, reinterpret_cast<unsigned long long*>(clocks), stream);
  if (e == hipSuccess)
    e = dap::launch_stage(g, w, dap::kAcceptAttention, DAP_STAGE_ATTENDED, stream);
  return hip_status(e);
}

dap_status dap_restore(const dap_config* cfg, const void* ws, size_t ws_bytes, void* out,
                       hipStream_t stream) {
  Geo g;
  dap_layout L;
  dap_status st = check_call(cfg, ws, ws_bytes, &g, &L);
  if (st != DAP_OK) return st;
  if (!out || !aligned(out)) return DAP_E_INVALID;
  return hip_status(dap::launch_restore(g, make_ws(const_cast<void*>(ws), L),
                                        static_cast<uint16_t*>(out), stream));
}

const char* dap_status_string(dap_status s) {
  switch (s) {
    case DAP_OK: return "ok";
    case DAP_E_INVALID: return "invalid argument";
    case DAP_E_UNSUPPORTED: return "unsupported configuration";
    case DAP_E_WORKSPACE: return "workspace too small";
    case DAP_E_HIP: return "HIP launch failure";
    case DAP_E_SCRATCH_LIMIT: return "batch * heads * head_dim exceeds the static scratch (65536)";
  }
  return "unknown status";
}

}  // extern "C"
