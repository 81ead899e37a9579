// C ABI of the block-sparse attention path: argument validation (before any
// HIP call), workspace carving and the launch sequence of every entry point.
// The operations themselves are documented in include/sparse_attn.h.
#include <math.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "sa_common.h"

// Work queue of sparse_attn_forward_noalloc, for callers that cannot
// allocate: one copy per device, held until the process ends.  Host code
// never uses this name as an address (on the host it is only a stand-in);
// it uses the device address looked up per device (scratch_address below).
static __device__ __align__(256) unsigned char scratch[SA_NOALLOC_SCRATCH_BYTES];

namespace sa {
bool attn_supported(int dtype, int d, int B);
}

namespace {

using sa::Dims;

constexpr int kMaxKB = 4096;
constexpr size_t kAlign = 256;

size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
// 32-bit element arrays (int32 CSR and demand arrays, mask words, fp32
// weights): NULL counts as aligned, its own check comes first
bool aligned4(const void* p) { return ((uintptr_t)p & 3u) == 0; }

// Validates the problem and fills the derived sizes.  No HIP call.
int check_problem(const sa_problem* p, Dims* g) {
  if (!p) return SA_ERR_INVALID_ARG;
  if (p->num_heads < 1) return SA_ERR_INVALID_ARG;
  if (p->dtype != SA_F32 && p->dtype != SA_BF16) return SA_ERR_INVALID_ARG;
  if (p->head_dim < 1 || p->block < 1) return SA_ERR_INVALID_ARG;
  if (p->head_dim != 64 && p->head_dim != 128) return SA_ERR_UNSUPPORTED;
  if (p->block != 64 && p->block != 128) return SA_ERR_UNSUPPORTED;
  const int64_t B = p->block;
  if (p->q_rows < B || p->q_rows % B || p->kv_rows < B || p->kv_rows % B) return SA_ERR_INVALID_ARG;
  if (p->q_valid <= p->q_rows - B || p->q_valid > p->q_rows) return SA_ERR_INVALID_ARG;
  if (p->kv_valid <= p->kv_rows - B || p->kv_valid > p->kv_rows) return SA_ERR_INVALID_ARG;
  const int64_t nqb = p->q_rows / B, nkb = p->kv_rows / B;
  if (nkb > kMaxKB) return SA_ERR_UNSUPPORTED;
  if ((int64_t)p->num_heads * nqb * nkb >= ((int64_t)1 << 31)) return SA_ERR_UNSUPPORTED;
  // work units are numbered 2 * item + half in 32 bits
  if ((int64_t)p->num_heads * nqb >= ((int64_t)1 << 30)) return SA_ERR_UNSUPPORTED;
  if ((int64_t)p->num_heads * p->kv_rows * p->head_dim >= ((int64_t)1 << 40)) return SA_ERR_UNSUPPORTED;
  if (p->select_mode != SA_TOP_P && p->select_mode != SA_TOP_K) return SA_ERR_INVALID_ARG;
  if (p->select_mode == SA_TOP_P && !(p->top_p > 0.f)) return SA_ERR_INVALID_ARG;
  if (p->select_mode == SA_TOP_P && p->top_k < 0) return SA_ERR_INVALID_ARG;
  if (p->select_mode == SA_TOP_K && p->top_k < 1) return SA_ERR_INVALID_ARG;
  if (p->score_mode != SA_SCORE_POOLED && p->score_mode != SA_SCORE_LOWRANK &&
      p->score_mode != SA_SCORE_LOWRANK_MAX && p->score_mode != SA_SCORE_LOWRANK_MASS)
    return SA_ERR_INVALID_ARG;
  if (p->score_mode != SA_SCORE_POOLED && (p->rank < 1 || p->rank > 64)) return SA_ERR_INVALID_ARG;
  if ((p->score_mode == SA_SCORE_LOWRANK_MAX || p->score_mode == SA_SCORE_LOWRANK_MASS) &&
      p->rank != 16)
    return SA_ERR_UNSUPPORTED;
  if (!isfinite(p->sm_scale) || !isfinite(p->score_scale)) return SA_ERR_INVALID_ARG;
  g->H = p->num_heads;
  g->d = p->head_dim;
  g->B = p->block;
  g->nqb = (int)nqb;
  g->nkb = (int)nkb;
  g->W = (int)((nkb + 31) / 32);
  g->rank = p->score_mode == SA_SCORE_LOWRANK ? p->rank : 0;
  g->score_mode = p->score_mode;
  g->q_rows = p->q_rows;
  g->q_valid = p->q_valid;
  g->kv_rows = p->kv_rows;
  g->kv_valid = p->kv_valid;
  g->dtype = p->dtype;
  return SA_OK;
}

// Workspace layout of every stage, in carve order.
struct SelectWs {
  size_t qbar, kbar, qt, kt, qtok, ktok, lse, scores, counts, total;
};
SelectWs select_ws(const Dims& g) {
  SelectWs w{};
  size_t o = 0;
  w.qbar = o; o += round_up(sizeof(double) * g.H * g.nqb * g.d);
  w.kbar = o; o += round_up(sizeof(double) * g.H * g.nkb * g.d);
  w.qt = o; o += round_up(sizeof(double) * g.H * g.nqb * g.rank);
  w.kt = o; o += round_up(sizeof(double) * g.H * g.nkb * g.rank);
  const bool token = g.score_mode == SA_SCORE_LOWRANK_MAX || g.score_mode == SA_SCORE_LOWRANK_MASS;
  const size_t tok = token ? 16 : 0;   // projected tokens: 16 fp64 components
  w.qtok = o; o += round_up(sizeof(double) * g.H * g.q_rows * tok);
  w.ktok = o; o += round_up(sizeof(double) * g.H * g.kv_rows * tok);
  // per query token and key block: ln of the predicted exp-sum (mass mode)
  const size_t lse_n = g.score_mode == SA_SCORE_LOWRANK_MASS ? (size_t)g.H * g.nkb * g.q_rows : 0;
  w.lse = o; o += round_up(sizeof(double) * lse_n);
  w.scores = o; o += round_up(sizeof(double) * g.H * g.nqb * g.nkb);
  w.counts = o; o += round_up(sizeof(int32_t) * g.H * g.nqb);
  w.total = o;
  return w;
}
size_t csr_ws(const Dims& g) { return round_up(sizeof(int32_t) * g.H * g.nqb); }
struct PackWs {
  size_t part, slot_of, total;
};
PackWs pack_ws(const Dims& g) {
  PackWs w{};
  size_t o = 0;
  w.part = o; o += round_up(sizeof(uint32_t) * g.H * sa::mark_groups(g) * g.W);
  w.slot_of = o; o += round_up(sizeof(int32_t) * g.H * g.nkb);
  w.total = o;
  return w;
}
size_t forward_ws(const Dims& g) { return round_up(sa::attn_ws_bytes(g)); }
struct BackwardWs {
  size_t delta, bits, counts, col_ptr, row_idx, order, total;
};
BackwardWs backward_ws(const Dims& g) {
  BackwardWs w{};
  size_t o = 0;
  w.delta = o; o += round_up(sizeof(float) * g.H * g.q_rows);
  w.bits = o; o += round_up(sizeof(uint32_t) * g.H * g.nqb * g.W);
  w.counts = o; o += round_up(sizeof(int32_t) * g.H * g.nkb);
  w.col_ptr = o; o += round_up(sizeof(int32_t) * (g.H * g.nkb + 1));
  w.row_idx = o; o += round_up(sizeof(int32_t) * (size_t)g.H * g.nqb * g.nkb);
  w.order = o; o += round_up(sizeof(int32_t) * g.H * g.nkb);
  w.total = o;
  return w;
}

// The fused pass needs the select stage's block means and projections only:
// the head of the select layout, up to the end of the key projections.
size_t fused_ctr(const Dims& g) {
  return select_ws(g).kt + round_up(sizeof(double) * g.H * g.nkb * g.rank);
}
size_t fused_ws(const Dims& g) { return fused_ctr(g) + round_up(sizeof(int32_t) * 8); }

size_t stage_bytes(const Dims& g, int stage) {
  switch (stage) {
    case SA_STAGE_FUSED: return fused_ws(g);
    case SA_STAGE_SELECT: return select_ws(g).total;
    case SA_STAGE_CSR: return csr_ws(g);
    case SA_STAGE_PACK: return pack_ws(g).total;
    case SA_STAGE_FORWARD: return forward_ws(g);
    case SA_STAGE_BACKWARD: return backward_ws(g).total;
  }
  return 0;
}

int check_ws(const Dims& g, int stage, void* ws, size_t ws_bytes) {
  const size_t need = stage_bytes(g, stage);
  if (need == 0) return SA_OK;
  if (!ws || ((uintptr_t)ws % kAlign)) return SA_ERR_INVALID_ARG;
  if (ws_bytes < need) return SA_ERR_WORKSPACE;
  return SA_OK;
}

#define SA_TRY_HIP(expr)                          \
  do {                                            \
    if ((expr) != hipSuccess) return SA_ERR_HIP;  \
  } while (0)

template <typename T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

// Device address of the current device's copy of `scratch`, looked up once
// per device (with that device current) and kept; NULL if the lookup fails.
constexpr int kMaxDevices = 64;
void* g_scratch_address[kMaxDevices];
std::mutex g_scratch_mutex;

void* scratch_address() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_address[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_scratch_address[dev] = p;
  }
  return g_scratch_address[dev];
}

// Pointer and size checks shared by the forward entry points.
int check_forward_args(const Dims& g, const void* q, const int32_t* row_ptr,
                       const int32_t* col_idx, const int32_t* col_slot, const void* k_src,
                       const void* v_src, const void* out, const float* lse_opt) {
  if (!sa::attn_supported(g.dtype, g.d, g.B)) return SA_ERR_UNSUPPORTED;
  if (!q || !row_ptr || !col_idx || !k_src || !v_src || !out) return SA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k_src) || !aligned16(v_src) || !aligned16(out))
    return SA_ERR_INVALID_ARG;
  if (!aligned4(lse_opt) || !aligned4(row_ptr) || !aligned4(col_idx) || !aligned4(col_slot))
    return SA_ERR_INVALID_ARG;
  return SA_OK;
}

}  // namespace

extern "C" {

int sa_abi_version(void) { return 8; }

const char* sa_status_string(int status) {
  switch (status) {
    case SA_OK: return "ok";
    case SA_ERR_INVALID_ARG: return "invalid argument (null pointer, bad size or misaligned buffer)";
    case SA_ERR_UNSUPPORTED: return "unsupported combination (head_dim, block, dtype or size)";
    case SA_ERR_WORKSPACE: return "workspace smaller than sa_workspace_size";
    case SA_ERR_HIP: return "HIP launch failed";
    case SA_ERR_CAPACITY: return "demand union exceeds the packed-buffer capacity";
    case SA_ERR_SCRATCH:
      return "problem needs more work-queue memory than the static scratch array of "
             "sparse_attn_forward_noalloc (SA_NOALLOC_SCRATCH_BYTES)";
  }
  return "unknown status";
}

int sa_workspace_size(const sa_problem* prob, int stage, size_t* bytes) {
  Dims g;
  if (!bytes) return SA_ERR_INVALID_ARG;
  const int st = check_problem(prob, &g);
  if (st != SA_OK) return st;
  if (stage < SA_STAGE_SELECT || stage > SA_STAGE_FUSED) return SA_ERR_INVALID_ARG;
  *bytes = stage_bytes(g, stage);
  return SA_OK;
}

int sparse_attn_select(const sa_problem* prob, const void* q, const void* k, const float* wq,
                       const float* wk, uint32_t* mask_bits, int32_t* row_ptr, int32_t* col_idx,
                       double* qbar_opt, double* kbar_opt, void* ws, size_t ws_bytes,
                       void* stream) {
  Dims g;
  int st = check_problem(prob, &g);
  if (st != SA_OK) return st;
  if (!q || !k || !mask_bits || !row_ptr || !col_idx) return SA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k)) return SA_ERR_INVALID_ARG;
  if (!aligned4(mask_bits) || !aligned4(row_ptr) || !aligned4(col_idx)) return SA_ERR_INVALID_ARG;
  if (g.score_mode != SA_SCORE_POOLED && (!wq || !wk)) return SA_ERR_INVALID_ARG;
  if (g.score_mode != SA_SCORE_POOLED && (!aligned4(wq) || !aligned4(wk))) return SA_ERR_INVALID_ARG;
  if ((qbar_opt && ((uintptr_t)qbar_opt & 7u)) || (kbar_opt && ((uintptr_t)kbar_opt & 7u)))
    return SA_ERR_INVALID_ARG;
  st = check_ws(g, SA_STAGE_SELECT, ws, ws_bytes);
  if (st != SA_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const SelectWs w = select_ws(g);
  double* qbar = qbar_opt ? qbar_opt : at<double>(ws, w.qbar);
  double* kbar = kbar_opt ? kbar_opt : at<double>(ws, w.kbar);
  double* qt = at<double>(ws, w.qt);
  double* kt = at<double>(ws, w.kt);
  double* scores = at<double>(ws, w.scores);
  int32_t* counts = at<int32_t>(ws, w.counts);

  SA_TRY_HIP(sa::launch_pool(g, q, k, wq, wk, qbar, kbar, qt, kt, s));
  if (g.score_mode == SA_SCORE_LOWRANK_MAX) {
    SA_TRY_HIP(sa::launch_lowrank_max(g, q, k, wq, wk, at<double>(ws, w.qtok),
                                      at<double>(ws, w.ktok), scores, s));
  } else if (g.score_mode == SA_SCORE_LOWRANK_MASS) {
    const double tau = prob->score_scale > 0.f ? (double)prob->score_scale : 1.0 / sqrt((double)g.d);
    SA_TRY_HIP(sa::launch_lowrank_mass(g, q, k, wq, wk, tau, at<double>(ws, w.qtok),
                                       at<double>(ws, w.ktok), at<double>(ws, w.lse), scores, s));
  } else if (g.rank > 0) {
    SA_TRY_HIP(sa::launch_scores(g, qt, kt, g.rank, 1.0, scores, s));
  } else {
    const double sc = prob->score_scale > 0.f ? (double)prob->score_scale : 1.0 / sqrt((double)g.d);
    SA_TRY_HIP(sa::launch_scores(g, qbar, kbar, g.d, sc, scores, s));
  }
  SA_TRY_HIP(sa::launch_select(g, scores, prob->select_mode, (double)prob->top_p, prob->top_k,
                               mask_bits, counts, s));
  SA_TRY_HIP(sa::launch_csr(g, mask_bits, counts, row_ptr, col_idx, s));
  return SA_OK;
}

int sparse_attn_csr_from_mask(const sa_problem* prob, const uint32_t* mask_bits, int32_t* row_ptr,
                              int32_t* col_idx, void* ws, size_t ws_bytes, void* stream) {
  Dims g;
  int st = check_problem(prob, &g);
  if (st != SA_OK) return st;
  if (!mask_bits || !row_ptr || !col_idx) return SA_ERR_INVALID_ARG;
  if (!aligned4(mask_bits) || !aligned4(row_ptr) || !aligned4(col_idx)) return SA_ERR_INVALID_ARG;
  st = check_ws(g, SA_STAGE_CSR, ws, ws_bytes);
  if (st != SA_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int32_t* counts = static_cast<int32_t*>(ws);
  SA_TRY_HIP(sa::launch_count_bits(g, mask_bits, counts, s));
  SA_TRY_HIP(sa::launch_csr(g, mask_bits, counts, row_ptr, col_idx, s));
  return SA_OK;
}

int kv_demand_pack(const sa_problem* prob, const int32_t* row_ptr, const int32_t* col_idx,
                   const void* k, const void* v, int32_t* demand_ptr, int32_t* demand_idx,
                   int32_t* col_slot, void* k_packed, void* v_packed, int64_t packed_cap_blocks,
                   int32_t* dev_status, void* ws, size_t ws_bytes, void* stream) {
  Dims g;
  int st = check_problem(prob, &g);
  if (st != SA_OK) return st;
  if (!row_ptr || !col_idx || !k || !v || !demand_ptr || !demand_idx || !col_slot || !dev_status)
    return SA_ERR_INVALID_ARG;
  if (packed_cap_blocks < 0) return SA_ERR_INVALID_ARG;
  if (packed_cap_blocks > 0 && (!k_packed || !v_packed)) return SA_ERR_INVALID_ARG;
  if (!aligned16(k) || !aligned16(v) || !aligned16(k_packed) || !aligned16(v_packed))
    return SA_ERR_INVALID_ARG;
  for (const void* p : {(const void*)row_ptr, (const void*)col_idx, (const void*)demand_ptr,
                        (const void*)demand_idx, (const void*)col_slot, (const void*)dev_status})
    if (!aligned4(p)) return SA_ERR_INVALID_ARG;
  st = check_ws(g, SA_STAGE_PACK, ws, ws_bytes);
  if (st != SA_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const PackWs w = pack_ws(g);
  int32_t* slot_of = at<int32_t>(ws, w.slot_of);
  SA_TRY_HIP(sa::launch_demand(g, row_ptr, col_idx, at<uint32_t>(ws, w.part), slot_of,
                               demand_ptr, demand_idx, packed_cap_blocks, dev_status, s));
  SA_TRY_HIP(sa::launch_pack(g, demand_ptr, demand_idx, k, v, k_packed, v_packed,
                             packed_cap_blocks, row_ptr, col_idx, slot_of, col_slot, s));
  return SA_OK;
}

// SA_SCHEDULE_AUTO resolved for this problem; -1 for an unknown schedule
static int resolve_schedule(const sa_problem* prob, int32_t schedule) {
  if (schedule == SA_SCHEDULE_AUTO)
    return prob->select_mode == SA_TOP_K ? SA_SCHEDULE_PER_UNIT : SA_SCHEDULE_PERSISTENT;
  return schedule == SA_SCHEDULE_PERSISTENT || schedule == SA_SCHEDULE_PER_UNIT ? schedule : -1;
}

int sa_forward_workgroups(const sa_problem* prob, int32_t schedule, int32_t* workgroups) {
  Dims g;
  const int st = check_problem(prob, &g);
  if (st != SA_OK) return st;
  if (!workgroups) return SA_ERR_INVALID_ARG;
  schedule = resolve_schedule(prob, schedule);
  if (schedule < 0) return SA_ERR_INVALID_ARG;
  if (!sa::attn_supported(g.dtype, g.d, g.B)) return SA_ERR_UNSUPPORTED;
  *workgroups = sa::attn_workgroups(g, schedule);
  return SA_OK;
}

int sparse_attn_forward_ex(const sa_problem* prob, const void* q, const int32_t* row_ptr,
                           const int32_t* col_idx, const int32_t* col_slot, const void* k_src,
                           const void* v_src, void* out, float* lse_opt, void* ws,
                           size_t ws_bytes, const sa_forward_opts* opts, void* stream) {
  Dims g;
  int st = check_problem(prob, &g);
  if (st != SA_OK) return st;
  st = check_forward_args(g, q, row_ptr, col_idx, col_slot, k_src, v_src, out, lse_opt);
  if (st != SA_OK) return st;
  int schedule = resolve_schedule(prob, opts ? opts->schedule : SA_SCHEDULE_AUTO);
  uint64_t* wg_clock = nullptr;
  if (schedule < 0) return SA_ERR_INVALID_ARG;
  if (opts) {
    if (opts->wg_clock && g.dtype == SA_BF16) {
      if (((uintptr_t)opts->wg_clock & 7u) || opts->clock_cap < sa::attn_workgroups(g, schedule))
        return SA_ERR_INVALID_ARG;
      wg_clock = opts->wg_clock;
    }
  }
  st = check_ws(g, SA_STAGE_FORWARD, ws, ws_bytes);
  if (st != SA_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const float sm = prob->sm_scale > 0.f ? prob->sm_scale : (float)(1.0 / sqrt((double)g.d));
  SA_TRY_HIP(sa::launch_attn(g, q, row_ptr, col_idx, col_slot, k_src, v_src, out, lse_opt, ws,
                             ws_bytes, sm, schedule, wg_clock, s));
  return SA_OK;
}

int sparse_attn_forward(const sa_problem* prob, const void* q, const int32_t* row_ptr,
                        const int32_t* col_idx, const int32_t* col_slot, const void* k_src,
                        const void* v_src, void* out, float* lse_opt, void* ws, size_t ws_bytes,
                        void* stream) {
  return sparse_attn_forward_ex(prob, q, row_ptr, col_idx, col_slot, k_src, v_src, out, lse_opt,
                                ws, ws_bytes, nullptr, stream);
}

int sparse_attn_fused(const sa_problem* prob, const void* q, const void* k, const void* v,
                      const float* wq, const float* wk, void* out, float* lse_opt,
                      uint32_t* mask_bits_opt, void* ws, size_t ws_bytes, void* stream) {
  Dims g;
  int st = check_problem(prob, &g);
  if (st != SA_OK) return st;
  if (g.dtype != SA_BF16 || g.d != 128 || g.B != 128 ||
      (g.score_mode != SA_SCORE_POOLED && g.score_mode != SA_SCORE_LOWRANK))
    return SA_ERR_UNSUPPORTED;
  if (!q || !k || !v || !out) return SA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return SA_ERR_INVALID_ARG;
  if (lse_opt && ((uintptr_t)lse_opt & 3u)) return SA_ERR_INVALID_ARG;
  if (mask_bits_opt && ((uintptr_t)mask_bits_opt & 3u)) return SA_ERR_INVALID_ARG;
  if (g.score_mode == SA_SCORE_LOWRANK && (!wq || !wk)) return SA_ERR_INVALID_ARG;
  if (g.score_mode == SA_SCORE_LOWRANK && (!aligned4(wq) || !aligned4(wk))) return SA_ERR_INVALID_ARG;
  st = check_ws(g, SA_STAGE_FUSED, ws, ws_bytes);
  if (st != SA_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const SelectWs w = select_ws(g);
  double* qbar = at<double>(ws, w.qbar);
  double* kbar = at<double>(ws, w.kbar);
  double* qt = at<double>(ws, w.qt);
  double* kt = at<double>(ws, w.kt);
  const float sm = prob->sm_scale > 0.f ? prob->sm_scale : (float)(1.0 / sqrt((double)g.d));
  SA_TRY_HIP(sa::launch_pool(g, q, k, wq, wk, qbar, kbar, qt, kt, s));
  if (g.rank > 0) {
    SA_TRY_HIP(sa::launch_fused(g, qt, kt, g.rank, 1.0, prob->select_mode, (double)prob->top_p,
                                prob->top_k, q, k, v, out, lse_opt, mask_bits_opt, sm,
                                at<int32_t>(ws, fused_ctr(g)), s));
  } else {
    const double sc = prob->score_scale > 0.f ? (double)prob->score_scale : 1.0 / sqrt((double)g.d);
    SA_TRY_HIP(sa::launch_fused(g, qbar, kbar, g.d, sc, prob->select_mode, (double)prob->top_p,
                                prob->top_k, q, k, v, out, lse_opt, mask_bits_opt, sm,
                                at<int32_t>(ws, fused_ctr(g)), s));
  }
  return SA_OK;
}

int sparse_attn_forward_noalloc(const sa_problem* prob, const void* q, const int32_t* row_ptr,
                                const int32_t* col_idx, const int32_t* col_slot,
                                const void* k_src, const void* v_src, void* out, float* lse_opt,
                                void* stream) {
  Dims g;
  int st = check_problem(prob, &g);
  if (st != SA_OK) return st;
  st = check_forward_args(g, q, row_ptr, col_idx, col_slot, k_src, v_src, out, lse_opt);
  if (st != SA_OK) return st;
  // whole items only: the queue is all the workspace the launch gets
  const size_t need = sa::attn_queue_ws_bytes(g);
  if (need > SA_NOALLOC_SCRATCH_BYTES) return SA_ERR_SCRATCH;
  void* ws = scratch_address();
  if (!ws) return SA_ERR_HIP;
  const float sm = prob->sm_scale > 0.f ? prob->sm_scale : (float)(1.0 / sqrt((double)g.d));
  SA_TRY_HIP(sa::launch_attn(g, q, row_ptr, col_idx, col_slot, k_src, v_src, out, lse_opt, ws,
                             need, sm, resolve_schedule(prob, SA_SCHEDULE_AUTO), nullptr,
                             static_cast<hipStream_t>(stream)));
  return SA_OK;
}

int sparse_attn_backward(const sa_problem* prob, const void* q, const void* k, const void* v,
                         const void* out, const void* dout, const float* lse,
                         const int32_t* row_ptr, const int32_t* col_idx, void* dq, void* dk,
                         void* dv, void* ws, size_t ws_bytes, void* stream) {
  Dims g;
  int st = check_problem(prob, &g);
  if (st != SA_OK) return st;
  if (g.dtype != SA_BF16 || !sa::attn_supported(g.dtype, g.d, g.B)) return SA_ERR_UNSUPPORTED;
  if (!q || !k || !v || !out || !dout || !lse || !row_ptr || !col_idx || !dq || !dk || !dv)
    return SA_ERR_INVALID_ARG;
  for (const void* p : {q, k, v, out, dout, (const void*)dq, (const void*)dk, (const void*)dv})
    if (!aligned16(p)) return SA_ERR_INVALID_ARG;
  if ((uintptr_t)lse & 15u) return SA_ERR_INVALID_ARG;
  if (!aligned4(row_ptr) || !aligned4(col_idx)) return SA_ERR_INVALID_ARG;
  st = check_ws(g, SA_STAGE_BACKWARD, ws, ws_bytes);
  if (st != SA_OK) return st;
  const BackwardWs w = backward_ws(g);
  const float sm = prob->sm_scale > 0.f ? prob->sm_scale : (float)(1.0 / sqrt((double)g.d));
  SA_TRY_HIP(sa::launch_backward(g, q, k, v, out, dout, lse, row_ptr, col_idx, dq, dk, dv,
                                 at<float>(ws, w.delta), at<uint32_t>(ws, w.bits),
                                 at<int32_t>(ws, w.counts),
                                 at<int32_t>(ws, w.col_ptr), at<int32_t>(ws, w.row_idx),
                                 at<int32_t>(ws, w.order), sm,
                                 static_cast<hipStream_t>(stream)));
  return SA_OK;
}

int sa_video_block_order(const sa_video_tiling* tiling, int64_t q_start, int64_t q_valid,
                         int32_t* kv_order, int32_t* kv_inverse, int32_t* q_order,
                         int32_t* q_inverse, void* stream) {
  if (!tiling || !kv_order || !kv_inverse || !q_order || !q_inverse) return SA_ERR_INVALID_ARG;
  const sa_video_tiling& t = *tiling;
  if (t.frames < 1 || t.height < 1 || t.width < 1) return SA_ERR_INVALID_ARG;
  if (t.tile_t < 1 || t.tile_h < 1 || t.tile_w < 1) return SA_ERR_INVALID_ARG;
  const int64_t n = (int64_t)t.frames * t.height * t.width;
  if (n >= ((int64_t)1 << 31)) return SA_ERR_UNSUPPORTED;
  if (q_start < 0 || q_valid < 1 || q_start + q_valid > n) return SA_ERR_INVALID_ARG;
  for (const void* p : {(const void*)kv_order, (const void*)kv_inverse, (const void*)q_order,
                        (const void*)q_inverse})
    if ((uintptr_t)p & 3u) return SA_ERR_INVALID_ARG;
  SA_TRY_HIP(sa::launch_video_order(t.frames, t.height, t.width, t.tile_t, t.tile_h, t.tile_w,
                                    q_start, q_valid, kv_order, kv_inverse, q_order, q_inverse,
                                    static_cast<hipStream_t>(stream)));
  return SA_OK;
}

int sa_permute_rows(int32_t heads, int64_t rows, int32_t row_bytes, const int32_t* idx,
                    const void* src, int64_t src_rows, void* dst, int64_t dst_rows,
                    void* stream) {
  if (heads < 1 || rows < 0 || src_rows < 0 || dst_rows < rows) return SA_ERR_INVALID_ARG;
  if (row_bytes < 4 || row_bytes > 65536 || row_bytes % 4) return SA_ERR_INVALID_ARG;
  if (!dst || (rows > 0 && (!idx || !src))) return SA_ERR_INVALID_ARG;
  if (((uintptr_t)dst & 3u) || ((uintptr_t)src & 3u) || ((uintptr_t)idx & 3u))
    return SA_ERR_INVALID_ARG;
  if ((int64_t)heads * std::max(src_rows, dst_rows) >= ((int64_t)1 << 40)) return SA_ERR_UNSUPPORTED;
  if (dst_rows == 0) return SA_OK;
  const bool wide = row_bytes % 16 == 0 && aligned16(src) && aligned16(dst);
  SA_TRY_HIP(sa::launch_permute_rows(heads, rows, row_bytes, idx, src, src_rows, dst, dst_rows,
                                     wide, static_cast<hipStream_t>(stream)));
  return SA_OK;
}

}  // extern "C"
