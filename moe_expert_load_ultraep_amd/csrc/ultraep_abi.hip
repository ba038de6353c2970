// C ABI of the exact-load rebalancing path: argument checks, plan-record
// layout, workspace sizing and kernel launches.  See include/ultraep.h for
// the contract of every entry point.
#include <hip/hip_runtime.h>

#include <climits>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <new>

#include "ultraep.h"
#include "ultraep_internal.h"

struct ultraep_ctx {
  ultraep::Shape sh;
};

namespace {

using ultraep::PlanLayout;
using ultraep::Shape;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

void build_layout(Shape* sh) {
  PlanLayout& L = sh->lay;
  const int32_t E = sh->E, R = sh->R, S = sh->S, P = sh->P;
  const int32_t len[ULTRAEP_PLAN_NUM_FIELDS] = {
      ultraep::kHeaderWords,  // header
      E,                      // counts
      E,                      // master quota
      R * S,                  // slot expert
      R * S,                  // slot quota
      P,                      // phys load
      P + 1,                  // phys off
      E + 1,                  // inst ptr
      E + R * S,              // inst phys
      E + R * S,              // inst end
      E + R * S,              // inst base
      R,                      // rank before
      R,                      // rank after
      E + R * S,              // inst local
  };
  int32_t at = 0;
  for (int f = 0; f < ULTRAEP_PLAN_NUM_FIELDS; ++f) {
    L.off[f] = at;
    L.len[f] = len[f];
    at += (len[f] + 3) & ~3;  // each field starts on a 16-byte boundary
  }
  L.words = (at + 63) & ~63;  // records are 256-byte multiples
}

// N = R*T*k pairs per layer, checked to fit int32.
int pairs_per_layer(const ultraep_ctx* ctx, int64_t T, int32_t k, int32_t* N) {
  if (T < 0 || k < 1 || k > ULTRAEP_MAX_TOPK || k > ctx->sh.E) return ULTRAEP_EINVAL;
  const int64_t n = static_cast<int64_t>(ctx->sh.R) * T * k;
  if (T > INT32_MAX || n > INT32_MAX) return ULTRAEP_EUNSUPPORTED;
  *N = static_cast<int32_t>(n);
  return ULTRAEP_OK;
}

int from_hip(hipError_t e) { return e == hipSuccess ? ULTRAEP_OK : ULTRAEP_ELAUNCH; }

// Workspace of ultraep_balance_static.  Every device the library runs on
// holds its own copy from the time the code object is loaded there until the
// process ends.  On the host the name is only a stand-in for the device
// symbol, never an address: host code takes the device address from
// hipGetSymbolAddress, looked up once per device on the first call there.
static __device__ __align__(256) unsigned char scratch[ULTRAEP_STATIC_WORKSPACE_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

// Device address of `scratch` on the current device.
int static_workspace(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return ULTRAEP_ELAUNCH;
  if (dev < 0 || dev >= kMaxDevices) return ULTRAEP_EUNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return ULTRAEP_ELAUNCH;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return ULTRAEP_OK;
}

// ultraep_balance with a caller's workspace, or (static_ws) with `scratch`.
// Every check runs before the workspace is looked up or anything launched.
int balance_impl(const ultraep_ctx* ctx, int32_t L, const int32_t* topk_idx, const float* topk_w,
                 int64_t T, int32_t k, void* workspace, size_t workspace_bytes, bool static_ws,
                 void* plans, int32_t* phys_idx, int32_t* pos, int32_t* inv, float* w_perm,
                 void* stream);

}  // namespace

extern "C" {

int ultraep_create(int32_t E, int32_t R, int32_t slots_per_rank, int32_t D,
                   const ultraep_options* opt, ultraep_ctx** out) {
  if (!out) return ULTRAEP_EINVAL;
  *out = nullptr;
  if (E < 1 || R < 1 || D < 1 || slots_per_rank < 0) return ULTRAEP_EINVAL;
  if (E % R != 0 || R % D != 0) return ULTRAEP_EINVAL;
  if (E > ULTRAEP_MAX_EXPERTS || E / R > ULTRAEP_MAX_MASTERS || slots_per_rank > ULTRAEP_MAX_SLOTS ||
      D > ULTRAEP_MAX_DOMAIN || static_cast<int64_t>(R) * slots_per_rank > ULTRAEP_MAX_TOTAL_SLOTS)
    return ULTRAEP_EUNSUPPORTED;
  ultraep_options o{1, 100, 0, 1, 1, ULTRAEP_REROUTE_RANGES, 1, 0};
  if (opt) {
    o = *opt;
    if ((o.replica_lean != 0 && o.replica_lean != 1) || o.min_tokens_per_replica < 0) return ULTRAEP_EINVAL;
    if (o.min_tokens_per_replica == 0) o.min_tokens_per_replica = 1;
    if (o.reroute_mode < ULTRAEP_REROUTE_RANGES || o.reroute_mode > ULTRAEP_REROUTE_INTERLEAVE)
      return ULTRAEP_EINVAL;
    if (o.eps_num < 0 || o.eps_den < 1 || (o.allow_zero_master != 0 && o.allow_zero_master != 1))
      return ULTRAEP_EINVAL;
    if (o.threshold_num == 0 && o.threshold_den == 0) o.threshold_num = o.threshold_den = 1;
    if (o.threshold_den < 1 || o.threshold_num < o.threshold_den ||
        static_cast<int64_t>(o.threshold_num) > 64ll * o.threshold_den)
      return ULTRAEP_EINVAL;
  }
  ultraep_ctx* c = new (std::nothrow) ultraep_ctx;
  if (!c) return ULTRAEP_EUNSUPPORTED;
  Shape& sh = c->sh;
  sh.E = E;
  sh.R = R;
  sh.S = slots_per_rank;
  sh.D = D;
  sh.M = E / R;
  sh.P = R * (sh.M + sh.S);
  sh.ndom = R / D;
  sh.n_inst = E + R * sh.S;
  sh.eps_num = o.eps_num;
  sh.eps_den = o.eps_den;
  sh.allow_zero = o.allow_zero_master;
  sh.thr_num = o.threshold_num;
  sh.thr_den = o.threshold_den;
  sh.reroute_mode = o.reroute_mode;
  sh.min_tokens = o.min_tokens_per_replica;
  sh.lean = o.replica_lean;
  build_layout(&sh);
  if (ultraep::plan_lds_bytes(sh) > 160 * 1024 || ultraep::rerouting_lds_bytes(sh, true) > 160 * 1024) {
    delete c;
    return ULTRAEP_EUNSUPPORTED;
  }
  *out = c;
  return ULTRAEP_OK;
}

int ultraep_destroy(ultraep_ctx* ctx) {
  delete ctx;
  return ULTRAEP_OK;
}

int ultraep_plan_bytes(const ultraep_ctx* ctx, size_t* out) {
  if (!ctx || !out) return ULTRAEP_EINVAL;
  *out = sizeof(int32_t) * static_cast<size_t>(ctx->sh.lay.words);
  return ULTRAEP_OK;
}

int ultraep_plan_field(const ultraep_ctx* ctx, int32_t field, size_t* offset_bytes, size_t* count) {
  if (!ctx || !offset_bytes || !count || field < 0 || field >= ULTRAEP_PLAN_NUM_FIELDS)
    return ULTRAEP_EINVAL;
  *offset_bytes = sizeof(int32_t) * static_cast<size_t>(ctx->sh.lay.off[field]);
  *count = static_cast<size_t>(ctx->sh.lay.len[field]);
  return ULTRAEP_OK;
}

int ultraep_workspace_bytes(const ultraep_ctx* ctx, int32_t L, int64_t T, int32_t k, size_t* out) {
  if (!ctx || !out || L < 0) return ULTRAEP_EINVAL;
  int32_t N = 0;
  const int st = pairs_per_layer(ctx, T, k, &N);
  if (st != ULTRAEP_OK) return st;
  const size_t ntiles = static_cast<size_t>(ultraep::ntiles_of(ctx->sh.R, static_cast<int64_t>(T) * k));
  *out = 2 * sizeof(int32_t) * static_cast<size_t>(L) * ntiles * static_cast<size_t>(ctx->sh.E);
  if (*out == 0) *out = 256;
  return ULTRAEP_OK;
}

int ultraep_balance(const ultraep_ctx* ctx, int32_t L, const int32_t* topk_idx,
                    const float* topk_w, int64_t T, int32_t k, void* workspace,
                    size_t workspace_bytes, void* plans, int32_t* phys_idx, int32_t* pos,
                    int32_t* inv, float* w_perm, void* stream) {
  return balance_impl(ctx, L, topk_idx, topk_w, T, k, workspace, workspace_bytes, false, plans,
                      phys_idx, pos, inv, w_perm, stream);
}

int ultraep_balance_static(const ultraep_ctx* ctx, int32_t L, const int32_t* topk_idx,
                           const float* topk_w, int64_t T, int32_t k, void* plans,
                           int32_t* phys_idx, int32_t* pos, int32_t* inv, float* w_perm,
                           void* stream) {
  return balance_impl(ctx, L, topk_idx, topk_w, T, k, nullptr, 0, true, plans, phys_idx, pos, inv,
                      w_perm, stream);
}

int ultraep_dispatch_layout(const ultraep_ctx* ctx, int32_t L, int64_t T, int32_t k,
                            const int32_t* pos, const float* topk_w, int32_t* inv, float* w_perm,
                            void* stream) {
  if (!ctx || L < 0) return ULTRAEP_EINVAL;
  int32_t N = 0;
  const int st = pairs_per_layer(ctx, T, k, &N);
  if (st != ULTRAEP_OK) return st;
  if (L == 0 || N == 0) return ULTRAEP_OK;
  if (!pos || !topk_w || !inv || !w_perm) return ULTRAEP_EINVAL;
  if (!aligned(pos, 4) || !aligned(topk_w, 4) || !aligned(inv, 4) || !aligned(w_perm, 4))
    return ULTRAEP_EUNSUPPORTED;
  return from_hip(
      ultraep::launch_layout(L, N, pos, topk_w, inv, w_perm, static_cast<hipStream_t>(stream)));
}

int ultraep_permute(const ultraep_ctx* ctx, const void* plan, const int32_t* inv, int32_t k,
                    const uint16_t* hidden, int64_t hidden_rows, int32_t H, int32_t p_begin,
                    int32_t p_end, uint16_t* out, int64_t out_capacity_rows, void* stream) {
  if (!ctx || !plan || !inv || !hidden || !out) return ULTRAEP_EINVAL;
  if (H <= 0 || k < 1 || k > ULTRAEP_MAX_TOPK || hidden_rows < 0 || out_capacity_rows < 0)
    return ULTRAEP_EINVAL;
  if (p_begin < 0 || p_end < p_begin || p_end > ctx->sh.P) return ULTRAEP_EINVAL;
  if (H % 8 != 0 || !aligned(hidden, 16) || !aligned(out, 16) || !aligned(inv, 4) ||
      !aligned(plan, 4))
    return ULTRAEP_EUNSUPPORTED;
  return from_hip(ultraep::launch_permute(ctx->sh, static_cast<const int32_t*>(plan), inv, k,
                                          hidden, hidden_rows, H, p_begin, p_end, out,
                                          out_capacity_rows, static_cast<hipStream_t>(stream)));
}

int ultraep_fold_grads(const ultraep_ctx* ctx, const void* plan, float* const* master_grads,
                       const float* replica_grads, int64_t numel, int32_t slot_begin,
                       int32_t slot_end, void* stream) {
  if (!ctx || !plan || !master_grads || numel < 0) return ULTRAEP_EINVAL;
  if (slot_begin < 0 || slot_end < slot_begin || slot_end > ctx->sh.R * ctx->sh.S)
    return ULTRAEP_EINVAL;
  if (slot_end > slot_begin && numel > 0 && !replica_grads) return ULTRAEP_EINVAL;
  if (!aligned(plan, 4) || !aligned(master_grads, 8) || !aligned(replica_grads, 4))
    return ULTRAEP_EUNSUPPORTED;
  return from_hip(ultraep::launch_fold(ctx->sh, static_cast<const int32_t*>(plan), master_grads,
                                       replica_grads, numel, slot_begin, slot_end,
                                       static_cast<hipStream_t>(stream)));
}

namespace {
// Shared checks of the combine calls: the token range and shapes.
int combine_checks(const ultraep_ctx* ctx, const int32_t* pos, int32_t k, const uint16_t* rows,
                   int64_t layout_rows, int32_t H, int64_t token_begin, int64_t token_end) {
  if (!ctx || !pos) return ULTRAEP_EINVAL;
  if (H <= 0 || k < 1 || k > ULTRAEP_MAX_TOPK || k > ctx->sh.E || layout_rows < 0) return ULTRAEP_EINVAL;
  if (token_begin < 0 || token_end < token_begin) return ULTRAEP_EINVAL;
  if (layout_rows > 0 && !rows) return ULTRAEP_EINVAL;
  if (H % 8 != 0 || layout_rows >= (int64_t{1} << 31) || token_end > (int64_t{1} << 40) / k ||
      !aligned(rows, 16) || !aligned(pos, 4))
    return ULTRAEP_EUNSUPPORTED;
  return ULTRAEP_OK;
}
}  // namespace

int ultraep_combine(const ultraep_ctx* ctx, const int32_t* pos, const float* topk_w, int32_t k,
                    const uint16_t* rows, int64_t layout_rows, int32_t H, int64_t token_begin,
                    int64_t token_end, uint16_t* out, void* stream) {
  const int st = combine_checks(ctx, pos, k, rows, layout_rows, H, token_begin, token_end);
  if (st != ULTRAEP_OK) return st;
  if (token_end > token_begin && !out) return ULTRAEP_EINVAL;
  if (!aligned(out, 16) || !aligned(topk_w, 4)) return ULTRAEP_EUNSUPPORTED;
  return from_hip(ultraep::launch_combine(pos, topk_w, k, rows, layout_rows, H, token_begin,
                                          token_end, out, static_cast<hipStream_t>(stream)));
}

int ultraep_combine_backward(const ultraep_ctx* ctx, const int32_t* pos, const float* topk_w,
                             int32_t k, const uint16_t* rows, int64_t layout_rows, int32_t H,
                             const uint16_t* grad_out, int64_t token_begin, int64_t token_end,
                             uint16_t* grad_rows, float* grad_topk_w, void* stream) {
  const int st = combine_checks(ctx, pos, k, rows, layout_rows, H, token_begin, token_end);
  if (st != ULTRAEP_OK) return st;
  if (token_end > token_begin && (!topk_w || !grad_out || !grad_topk_w)) return ULTRAEP_EINVAL;
  if (token_end > token_begin && layout_rows > 0 && !grad_rows) return ULTRAEP_EINVAL;
  if (!aligned(grad_out, 16) || !aligned(grad_rows, 16) || !aligned(topk_w, 4) ||
      !aligned(grad_topk_w, 4))
    return ULTRAEP_EUNSUPPORTED;
  return from_hip(ultraep::launch_combine_backward(pos, topk_w, k, rows, layout_rows, H, grad_out,
                                                   token_begin, token_end, grad_rows, grad_topk_w,
                                                   static_cast<hipStream_t>(stream)));
}

int ultraep_weight_sync_plan(const ultraep_ctx* ctx, const void* plan, const ultraep_relay_options* opt,
                             int32_t* relay, void* stream) {
  if (!ctx || !plan || !relay) return ULTRAEP_EINVAL;
  ultraep_relay_options o{ULTRAEP_RELAY_ADAPTIVE, 4, 8, 2, ctx->sh.D, {0, 0, 0}};
  if (opt) {
    o = *opt;
    for (int32_t r : o.reserved)
      if (r != 0) return ULTRAEP_EINVAL;
  }
  if (o.mode < ULTRAEP_RELAY_DIRECT || o.mode > ULTRAEP_RELAY_FORCE || o.min_replicas < 0 ||
      o.max_relays < 0 || o.min_gain < 0 || o.domain_gpus < 0)
    return ULTRAEP_EINVAL;
  if (!aligned(plan, 4) || !aligned(relay, 4)) return ULTRAEP_EUNSUPPORTED;
  return from_hip(ultraep::launch_relay_plan(ctx->sh, static_cast<const int32_t*>(plan), o.mode,
                                             o.min_replicas, o.max_relays, o.min_gain, o.domain_gpus,
                                             relay, static_cast<hipStream_t>(stream)));
}

int ultraep_weight_sync(const ultraep_ctx* ctx, const void* plan, const uint16_t* const* master_weights,
                        uint16_t* replica_weights, int64_t numel, int32_t slot_begin, int32_t slot_end,
                        const int32_t* relay, void* stream) {
  if (!ctx || !plan || !master_weights || numel < 0) return ULTRAEP_EINVAL;
  const int32_t all = ctx->sh.R * ctx->sh.S;
  if (slot_begin < 0 || slot_end < slot_begin || slot_end > all) return ULTRAEP_EINVAL;
  if (slot_end > slot_begin && numel > 0 && !replica_weights) return ULTRAEP_EINVAL;
  if (relay && (slot_begin != 0 || slot_end != all)) return ULTRAEP_EINVAL;
  if (!aligned(plan, 4) || !aligned(master_weights, 8) || !aligned(replica_weights, 2) ||
      !aligned(relay, 4))
    return ULTRAEP_EUNSUPPORTED;
  return from_hip(ultraep::launch_weight_sync(ctx->sh, static_cast<const int32_t*>(plan), master_weights,
                                              replica_weights, numel, slot_begin, slot_end, relay,
                                              static_cast<hipStream_t>(stream)));
}

const char* ultraep_status_string(int status) {
  switch (status) {
    case ULTRAEP_OK: return "ok";
    case ULTRAEP_EINVAL: return "invalid argument";
    case ULTRAEP_EUNSUPPORTED: return "unsupported shape, size or alignment";
    case ULTRAEP_ELAUNCH: return "HIP launch or runtime error";
    case ULTRAEP_EWORKSPACE: return "workspace too small";
    case ULTRAEP_ESCRATCH: return "needs more than the static workspace";
    default: return "unknown status";
  }
}

}  // extern "C"

namespace {

int balance_impl(const ultraep_ctx* ctx, int32_t L, const int32_t* topk_idx, const float* topk_w,
                 int64_t T, int32_t k, void* workspace, size_t workspace_bytes, bool static_ws,
                 void* plans, int32_t* phys_idx, int32_t* pos, int32_t* inv, float* w_perm,
                 void* stream) {
  if (!ctx || L < 0) return ULTRAEP_EINVAL;
  int32_t N = 0;
  int st = pairs_per_layer(ctx, T, k, &N);
  if (st != ULTRAEP_OK) return st;
  if (L == 0) return ULTRAEP_OK;
  if (!plans || (!static_ws && !workspace)) return ULTRAEP_EINVAL;
  if (N > 0 && (!topk_idx || !phys_idx || !pos)) return ULTRAEP_EINVAL;
  const bool layout = inv || w_perm || topk_w;
  if (layout && N > 0 && (!inv || !w_perm || !topk_w)) return ULTRAEP_EINVAL;
  if (!aligned(topk_idx, 4) || !aligned(phys_idx, 4) || !aligned(pos, 4) || !aligned(plans, 4) ||
      !aligned(workspace, 4) || !aligned(topk_w, 4) || !aligned(inv, 4) || !aligned(w_perm, 4))
    return ULTRAEP_EUNSUPPORTED;
  size_t need = 0;
  st = ultraep_workspace_bytes(ctx, L, T, k, &need);
  if (st != ULTRAEP_OK) return st;
  if (static_ws) {
    if (need > ULTRAEP_STATIC_WORKSPACE_BYTES) return ULTRAEP_ESCRATCH;
    st = static_workspace(&workspace);
    if (st != ULTRAEP_OK) return st;
  } else if (workspace_bytes < need) {
    return ULTRAEP_EWORKSPACE;
  }
  return from_hip(ultraep::launch_balance(ctx->sh, L, topk_idx, topk_w, static_cast<int32_t>(T * k),
                                          static_cast<int32_t*>(workspace),
                                          static_cast<int32_t*>(plans), phys_idx, pos,
                                          layout ? inv : nullptr, w_perm,
                                          static_cast<hipStream_t>(stream)));
}

}  // namespace
