// C ABI of libmoe_mi355x.so (declared in include/moe.h): argument validation,
// capacity, workspace carving and the launch sequence of the forward pass.
// All device work is enqueued on the caller's stream; nothing here
// synchronises except moe_profile_read().
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <atomic>
#include <mutex>
#include <string>
#include <vector>

#include "common.h"
#include "launch.h"
#include "plan.h"

namespace moe {

// ---------------------------------------------------------------- profiling
namespace {
struct ProfRec {
  const char* name;
  hipEvent_t e0, e1;
};
std::mutex g_prof_mu;
std::atomic<bool> g_prof_on{false};   // read by every launch, set under the mutex
std::vector<ProfRec> g_prof_recs;
std::vector<hipEvent_t> g_prof_pool;
uint32_t g_prof_gen = 0;          // generation of g_prof_recs (under the mutex)

hipEvent_t prof_event() {
  if (!g_prof_pool.empty()) {
    hipEvent_t e = g_prof_pool.back();
    g_prof_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}
}  // namespace

// A handle is the record's index in the low 32 bits and the generation of
// the record list (bumped whenever moe_profile_enable / moe_profile_read
// clear it) above them, so an end event never lands on another launch's
// record or on a list that was cleared in between.
int64_t prof_before(const char* name, hipStream_t s) {
  if (!g_prof_on.load(std::memory_order_relaxed)) return -1;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  ProfRec r{name, prof_event(), prof_event()};
  if (!r.e0 || !r.e1) return -1;
  hipEventRecord(r.e0, s);
  g_prof_recs.push_back(r);
  return ((int64_t)g_prof_gen << 32) | (int64_t)(g_prof_recs.size() - 1);
}

void prof_after(int64_t rec, hipStream_t s) {
  if (rec < 0) return;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  const uint32_t gen = (uint32_t)(rec >> 32);
  const size_t i = (size_t)(rec & 0xffffffff);
  if (gen == g_prof_gen && i < g_prof_recs.size()) hipEventRecord(g_prof_recs[i].e1, s);
}

int cu_count() {
  // per device, filled on first use (threads racing here store the same value)
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

}  // namespace moe

using namespace moe;

namespace {

constexpr size_t ALIGN = 256;
size_t up(size_t v) { return (v + ALIGN - 1) / ALIGN * ALIGN; }

bool al(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

size_t esize(const moe_config_t* c) { return c->dtype == MOE_BF16 ? 2 : 4; }

moe_status_t check_cfg(const moe_config_t* c, int64_t T) {
  if (!c || T < 0) return MOE_ERR_INVALID_ARG;
  if (c->d <= 0 || c->num_experts < 1 || c->top_k < 1 || c->top_k > c->num_experts ||
      c->d_ff <= 0 || c->num_shared < 0)
    return MOE_ERR_INVALID_ARG;
  if (c->act < MOE_ACT_RELU || c->act > MOE_ACT_SWIGLU) return MOE_ERR_INVALID_ARG;
  if (c->gating < MOE_GATE_SOFTMAX_TOPK || c->gating > MOE_GATE_SOFTMAX_FULL)
    return MOE_ERR_INVALID_ARG;
  if (c->dtype != MOE_F32 && c->dtype != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (isnan(c->capacity_factor)) return MOE_ERR_INVALID_ARG;
  if (c->capacity_priority != MOE_PRIORITY_TOKEN && c->capacity_priority != MOE_PRIORITY_SLOT)
    return MOE_ERR_INVALID_ARG;
  if (c->num_shared > 0 && c->d_ff_shared <= 0) return MOE_ERR_INVALID_ARG;
  if (c->num_experts > 256 || c->top_k > 16 || c->num_shared > 8) return MOE_ERR_UNSUPPORTED;
  const int q = c->dtype == MOE_BF16 ? 64 : 4;
  if (c->d % q || c->d_ff % q || (c->num_shared > 0 && c->d_ff_shared % q))
    return MOE_ERR_UNSUPPORTED;
  if (T * (int64_t)c->top_k > (int64_t)1 << 30) return MOE_ERR_UNSUPPORTED;
  if (c->num_shared > 0 && T * (int64_t)c->num_shared > (int64_t)1 << 30) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

int64_t capacity_of(const moe_config_t* c, int64_t T) {
  const double rho = (double)c->capacity_factor;
  if (!(rho > 0.0)) return -1;
  return (int64_t)floor(((rho * (double)c->top_k) * (double)T) / (double)c->num_experts);
}

bool small_batch(int64_t rows) { return rows <= MOE_DECODE_MAX_ROWS; }

struct PermWs {
  size_t block_counts, kept_total, total;
};
PermWs perm_ws(const moe_config_t* c, int64_t T) {
  PermWs w;
  size_t o = 0;
  w.block_counts = o;
  o += up((size_t)permute_nblocks(T * c->top_k) * c->num_experts * 4);
  w.kept_total = o;
  o += up(4);
  w.total = o;
  return w;
}

struct FfnWs {
  size_t H, Hs, plan1, plan2, plan3, plan4, part, total;
  int split;   // K parts of the routed second GEMM
};
FfnWs ffn_ws(const moe_config_t* c, int64_t T) {
  FfnWs w;
  const int64_t R = T * c->top_k;
  const int S = c->num_shared;
  size_t o = 0;
  w.H = o;
  o += up((size_t)R * c->d_ff * esize(c));
  w.Hs = o;
  o += up((size_t)S * T * (S ? c->d_ff_shared : 0) * esize(c));
  w.split = ffn_split(R, c->num_experts, c->d, c->d_ff, small_batch(R), c->dtype);
  w.plan1 = o;
  o += ffn_plan_bytes(R, c->num_experts, c->d_ff, small_batch(R), c->dtype);
  w.plan2 = o;
  o += ffn_plan_bytes(R, c->num_experts, c->d, small_batch(R), c->dtype, w.split);
  w.part = o;   // fp32 partial tiles of the second GEMM's tail split
  if (w.split > 1) o += up((size_t)kTailParts * 256 * 256 * 4);
  w.plan3 = w.plan4 = o;
  if (S) {
    o += ffn_plan_bytes((int64_t)S * T, S, c->d_ff_shared, small_batch(T), c->dtype);
    w.plan4 = o;
    o += ffn_plan_bytes((int64_t)S * T, S, c->d, small_batch(T), c->dtype);
  }
  w.total = o;
  return w;
}

struct FwdWs {
  size_t idx, gate, counts, dropped, offsets, perm_src, slot_pos, eout, sout, route, perm, ffn,
      stats, total;
};
FwdWs fwd_ws(const moe_config_t* c, int64_t T) {
  FwdWs w;
  const int64_t R = T * c->top_k;
  size_t o = 0;
  w.idx = o; o += up((size_t)R * 4);
  w.gate = o; o += up((size_t)R * 4);
  w.counts = o; o += up((size_t)c->num_experts * 4);
  w.dropped = o; o += up(4);
  w.offsets = o; o += up((size_t)(c->num_experts + 1) * 4);
  w.perm_src = o; o += up((size_t)R * 4);
  w.slot_pos = o; o += up((size_t)R * 4);
  w.eout = o; o += up((size_t)R * c->d * esize(c));
  w.sout = o; o += up((size_t)c->num_shared * T * c->d * esize(c));
  w.route = o; o += up(route_ws_bytes(T, c->num_experts, c->dtype));
  w.perm = o; o += perm_ws(c, T).total;
  w.ffn = o; o += ffn_ws(c, T).total;
  w.stats = o; o += up(stats_ws_bytes(T, c->num_experts));
  w.total = o;
  return w;
}

// Training forward: the forward's workspace followed by what the backward
// reads besides it (scores, gathered rows, pre-activations).
struct TrainWs {
  FwdWs fwd;
  size_t logits, x_perm, save1, save2, ssave1, ssave2, total;
};
TrainWs train_ws(const moe_config_t* c, int64_t T) {
  TrainWs w;
  w.fwd = fwd_ws(c, T);
  const int64_t R = T * c->top_k;
  const int64_t ST = (int64_t)c->num_shared * T;
  const bool glu = c->act == MOE_ACT_SWIGLU;
  size_t o = w.fwd.total;
  w.logits = o; o += up((size_t)T * c->num_experts * 4);
  w.x_perm = o; o += up((size_t)R * c->d * 2);
  w.save1 = o; o += up((size_t)R * c->d_ff * 2);
  w.save2 = o; o += glu ? up((size_t)R * c->d_ff * 2) : 0;
  w.ssave1 = o; o += up((size_t)ST * (ST ? c->d_ff_shared : 0) * 2);
  w.ssave2 = o; o += up((size_t)ST * (ST ? c->d_ff_shared : 0) * 2);
  w.total = o;
  return w;
}

constexpr size_t kZeroBytes = 4096;

int64_t bwd_entries(int64_t rows, int G, int N) {
  const int BM = bwd_tile_rows(), BN = bwd_tile_cols();
  int64_t mt = (rows + BM - 1) / BM + G;
  if (mt > rows) mt = rows;
  return mt * ((N + BN - 1) / BN);
}
// extra: entries beyond the row tiles (a tail split's K parts)
size_t bwd_plan_bytes(int64_t rows, int G, int N, int extra = 0) {
  return up(kPlanHeader + 16 * ((size_t)bwd_entries(rows, G, N) + (size_t)extra));
}

// 2 when the routed dX GEMM may split its partial last round of tiles over K
// (both operand pairs for SwiGLU), else 1
int dx_split(const moe_config_t* c, int64_t T) {
  const int K_all = c->d_ff * (c->act == MOE_ACT_SWIGLU ? 2 : 1);
  return bwd_dx_split(T * c->top_k, c->num_experts, c->d, K_all);
}

struct BwdWs {
  size_t zero, dO, dG, dU, dXp, dXpart, dlogits, dGs, dUs, dXs, plan_h, plan_x, splan_h, splan_x,
      wr, order, total;
  int split;       // 2: the routed dX GEMM may run its tail tiles in K parts
};
BwdWs bwd_ws(const moe_config_t* c, int64_t T) {
  BwdWs w;
  const int64_t R = T * c->top_k;
  const int S = c->num_shared;
  const int64_t ST = (int64_t)S * T;
  const bool glu = c->act == MOE_ACT_SWIGLU;
  size_t o = 0;
  w.zero = o; o += kZeroBytes;
  w.dO = o; o += up((size_t)R * c->d * 2);
  w.dG = o; o += up((size_t)R * c->d_ff * 2);
  w.dU = o; o += glu ? up((size_t)R * c->d_ff * 2) : 0;
  w.split = dx_split(c, T);
  w.dXp = o; o += up((size_t)R * c->d * 2);
  w.dXpart = o; o += w.split > 1 ? up((size_t)kTailParts * 256 * 256 * 4) : 0;
  w.dlogits = o; o += up((size_t)T * c->num_experts * 4);
  w.dGs = o; o += up((size_t)ST * (S ? c->d_ff_shared : 0) * 2);
  w.dUs = o; o += up((size_t)ST * (S ? c->d_ff_shared : 0) * 2);
  w.dXs = o; o += up((size_t)ST * c->d * 2);
  w.plan_h = o; o += bwd_plan_bytes(R, c->num_experts, c->d_ff);
  w.plan_x = o; o += bwd_plan_bytes(R, c->num_experts, c->d, w.split > 1 ? kTailParts : 0);
  w.splan_h = w.splan_x = o;
  if (S) {
    o += bwd_plan_bytes(ST, S, c->d_ff_shared);
    w.splan_x = o;
    o += bwd_plan_bytes(ST, S, c->d);
  }
  w.wr = o; o += up(wr_ws_bytes(T, c->num_experts, c->d));
  w.order = o; o += up((size_t)(c->num_experts + 8) * 4);
  w.total = o;
  return w;
}

char* at(void* base, size_t off) { return static_cast<char*>(base) + off; }
const char* at(const void* base, size_t off) { return static_cast<const char*>(base) + off; }

moe_status_t hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

RouteArgs route_args(const moe_config_t* c, int64_t T, const void* x, const void* wr,
                     const float* off, const float* bias, float* logits, int32_t* idx,
                     float* gate, void* ws) {
  return RouteArgs{x, wr, off, bias, logits, idx, gate, static_cast<float*>(ws), T, c->d,
                   c->num_experts, c->top_k, c->gating, c->dtype};
}

moe_status_t do_route(const moe_config_t* c, int64_t T, const void* x, const void* wr,
                      const float* off, const float* bias, float* logits, int32_t* idx,
                      float* gate, void* ws, hipStream_t s) {
  return hip_status(launch_route(route_args(c, T, x, wr, off, bias, logits, idx, gate, ws), s));
}

PermuteArgs permute_args(const moe_config_t* c, int64_t T, const int32_t* idx, const void* x,
                         int32_t* counts, int32_t* offsets, int32_t* perm_src,
                         int32_t* slot_pos, int32_t* dropped, void* x_perm, void* ws,
                         const PlanSpec* plans) {
  const PermWs w = perm_ws(c, T);
  PermuteArgs a;
  a.topk_idx = idx;
  a.x = x;
  a.counts = counts;
  a.offsets = offsets;
  a.perm_src = perm_src;
  a.slot_pos = slot_pos;
  a.num_dropped = dropped;
  a.x_perm = x_perm;
  a.block_counts = reinterpret_cast<int32_t*>(at(ws, w.block_counts));
  a.kept_total = reinterpret_cast<int32_t*>(at(ws, w.kept_total));
  a.T = T;
  a.k = c->top_k;
  a.E = c->num_experts;
  a.d = c->d;
  a.dtype = c->dtype;
  a.capacity = capacity_of(c, T);
  a.slot_major = c->capacity_priority == MOE_PRIORITY_SLOT ? 1 : 0;
  a.plans = plans;
  return a;
}

moe_status_t do_permute(const moe_config_t* c, int64_t T, const int32_t* idx, const void* x,
                        int32_t* counts, int32_t* offsets, int32_t* perm_src,
                        int32_t* slot_pos, int32_t* dropped, void* x_perm, void* ws,
                        hipStream_t s, const PlanSpec* plans = nullptr,
                        bool* plans_built = nullptr) {
  const PermuteArgs a = permute_args(c, T, idx, x, counts, offsets, perm_src, slot_pos, dropped,
                                     x_perm, ws, plans);
  return hip_status(launch_permute(a, s, plans_built));
}

// The GEMM passes of the routed experts (p, p2) and of the shared experts
// (q, q2).  x_perm may be null when perm_src is given: the first GEMM then
// reads the rows of x through perm_src (row gather folded into its loads).
struct FfnPasses {
  FfnPassArgs p, p2, q, q2;
  bool shared;
};

FfnPasses ffn_passes(const moe_config_t* c, int64_t T, const void* x, const void* x_perm,
                     const int32_t* perm_src, const int32_t* offsets, const void* w1,
                     const void* w3, const void* w2, const void* ws1, const void* ws3,
                     const void* ws2, void* eout, void* sout, void* ws,
                     const TrainWs* train = nullptr, void* saved = nullptr) {
  const FfnWs w = ffn_ws(c, T);
  const int64_t R = T * c->top_k;
  const int mode1 = c->act == MOE_ACT_SWIGLU ? 3 : (c->act == MOE_ACT_GELU ? 2 : 1);
  FfnPasses f;
  memset(&f, 0, sizeof(f));
  FfnPassArgs& p = f.p;
  p.A = x_perm ? x_perm : x;
  p.a_rows = x_perm ? nullptr : perm_src;
  p.a_div = c->top_k;
  p.w = w1;
  p.w_up = c->act == MOE_ACT_SWIGLU ? w3 : nullptr;
  p.C = at(ws, w.H);
  p.seg_offsets = offsets;
  p.G = c->num_experts;
  p.K = c->d;
  p.N = c->d_ff;
  p.mode = mode1;
  p.dtype = c->dtype;
  p.plan = at(ws, w.plan1);
  p.max_rows = R;
  p.small = small_batch(R);
  if (train) {
    p.save1 = at(saved, train->save1);
    p.save2 = c->act == MOE_ACT_SWIGLU ? at(saved, train->save2) : nullptr;
  }
  FfnPassArgs& p2 = f.p2;
  p2 = p;
  p2.A = at(ws, w.H);
  p2.a_rows = nullptr;
  p2.w = w2;
  p2.w_up = nullptr;
  p2.C = eout;
  p2.K = c->d_ff;
  p2.N = c->d;
  p2.mode = 0;
  p2.plan = at(ws, w.plan2);
  p2.save1 = p2.save2 = nullptr;
  p2.split = w.split;
  p2.part = w.split > 1 ? reinterpret_cast<float*>(at(ws, w.part)) : nullptr;
  f.shared = c->num_shared > 0;
  if (f.shared) {
    const int S = c->num_shared;
    FfnPassArgs& q = f.q;
    q.A = x;
    q.w = ws1;
    q.w_up = ws3;
    q.C = at(ws, w.Hs);
    q.seg_offsets = nullptr;
    q.dense_rows = T;
    q.G = S;
    q.K = c->d;
    q.N = c->d_ff_shared;
    q.mode = 3;
    q.dtype = c->dtype;
    q.a_seg_rows = 0;
    q.c_seg_rows = T;
    q.plan = at(ws, w.plan3);
    q.max_rows = (int64_t)S * T;
    q.small = small_batch(T);
    if (train) {
      q.save1 = at(saved, train->ssave1);
      q.save2 = at(saved, train->ssave2);
    }
    FfnPassArgs& q2 = f.q2;
    q2 = q;
    q2.A = at(ws, w.Hs);
    q2.w = ws2;
    q2.w_up = nullptr;
    q2.C = sout;
    q2.K = c->d_ff_shared;
    q2.N = c->d;
    q2.mode = 0;
    q2.a_seg_rows = T;
    q2.plan = at(ws, w.plan4);
    q2.split = 1;
    q2.part = nullptr;
    q2.save1 = q2.save2 = nullptr;
  }
  return f;
}

// routed_plans_built: the permutation already wrote the routed experts' plans
moe_status_t run_ffn(const FfnPasses& f, bool routed_plans_built, hipStream_t s) {
  if (!routed_plans_built && launch_ffn_plans(f.p, f.p2, s) != hipSuccess) return MOE_ERR_HIP;
  if (launch_ffn_pass(f.p, s) != hipSuccess) return MOE_ERR_HIP;
  if (launch_ffn_pass(f.p2, s) != hipSuccess) return MOE_ERR_HIP;
  if (launch_ffn_tail_reduce(f.p2, s) != hipSuccess) return MOE_ERR_HIP;
  if (f.shared) {
    if (launch_ffn_plans(f.q, f.q2, s) != hipSuccess) return MOE_ERR_HIP;
    if (launch_ffn_pass(f.q, s) != hipSuccess) return MOE_ERR_HIP;
    if (launch_ffn_pass(f.q2, s) != hipSuccess) return MOE_ERR_HIP;
  }
  return MOE_OK;
}

// The stepwise entry point: expert_out in bf16.
moe_status_t do_ffn(const moe_config_t* c, int64_t T, const void* x, const void* x_perm,
                    const int32_t* perm_src, const int32_t* offsets, const void* w1,
                    const void* w3, const void* w2, const void* ws1, const void* ws3,
                    const void* ws2, void* eout, void* sout, void* ws, hipStream_t s) {
  const FfnPasses f =
      ffn_passes(c, T, x, x_perm, perm_src, offsets, w1, w3, w2, ws1, ws3, ws2, eout, sout, ws);
  return run_ffn(f, false, s);
}

moe_status_t do_combine(const moe_config_t* c, int64_t T, const void* eout,
                        const int32_t* slot_pos, const float* gate, const void* sout, void* y,
                        hipStream_t s) {
  CombineArgs a{eout, slot_pos, gate, sout, y, T, c->top_k, c->d,
                sout ? c->num_shared : 0, c->dtype};
  return hip_status(launch_combine(a, s));
}

// ------------------------------------------------- allocation-free forward
// The workspace of moe_forward_noalloc: one file-scope device array per GPU
// (the HIP runtime places a copy on each device the library runs on, held
// until the process ends).  Host code never uses the array's name as an
// address: it is a host-side stand-in.  The device address comes from
// hipGetSymbolAddress, once per device with that device current, and is
// kept per device.  Nothing in it needs to start at zero: every kernel of
// the forward pass writes what it later reads within the same call (plan
// queue words and the router's done-counter are reset by the kernels that
// precede their readers).
constexpr size_t kScratchBytes = MOE_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_addr[kMaxDevices];
std::mutex g_scratch_mu;

// This device's address of the scratch array, or null on a HIP error.
void* scratch_ptr() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  p = g_scratch_addr[dev].load(std::memory_order_relaxed);
  if (!p) {
    void* q = nullptr;
    if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || !q) return nullptr;
    g_scratch_addr[dev].store(q, std::memory_order_release);
    p = q;
  }
  return p;
}

// moe_forward, and with use_scratch the allocation-free variant: the
// workspace is then this device's file-scope scratch array.
moe_status_t forward_impl(const moe_config_t* cfg, int64_t T, const void* x,
                          const void* w_router, const float* logit_offset,
                          const float* select_bias, const void* w1, const void* w3,
                          const void* w2, const void* ws1, const void* ws3, const void* ws2,
                          void* y, int32_t* topk_idx, float* topk_gate, int32_t* expert_counts,
                          int32_t* num_dropped, void* workspace, size_t ws_bytes, void* stream,
                          bool use_scratch) {
  moe_status_t st = check_cfg(cfg, T);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;  // nothing to do; token-sized pointers may be null
  if (!x || !w_router || !w1 || !w2 || !y) return MOE_ERR_INVALID_ARG;
  if (cfg->act == MOE_ACT_SWIGLU && !w3) return MOE_ERR_INVALID_ARG;
  if (cfg->num_shared > 0 && (!ws1 || !ws3 || !ws2)) return MOE_ERR_INVALID_ARG;
  const void* p16[] = {x, w_router, w1, w2, y, w3, ws1, ws3, ws2};
  for (const void* p : p16)
    if (p && !al(p, 16)) return MOE_ERR_INVALID_ARG;
  const void* p4[] = {logit_offset, select_bias, topk_idx, topk_gate, expert_counts, num_dropped};
  for (const void* p : p4)
    if (p && !al(p, 4)) return MOE_ERR_INVALID_ARG;
  const FwdWs w = fwd_ws(cfg, T);
  if (use_scratch) {
    // sized before any HIP call: a batch beyond the array is refused
    if (w.total > kScratchBytes) return MOE_ERR_WORKSPACE;
    workspace = scratch_ptr();
    if (!workspace) return MOE_ERR_HIP;
    ws_bytes = kScratchBytes;
  }
  if (!workspace || !al(workspace, ALIGN)) return MOE_ERR_INVALID_ARG;
  if (ws_bytes < w.total) return MOE_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int32_t* idx = topk_idx ? topk_idx : reinterpret_cast<int32_t*>(at(workspace, w.idx));
  float* gate = topk_gate ? topk_gate : reinterpret_cast<float*>(at(workspace, w.gate));
  int32_t* counts = expert_counts ? expert_counts : reinterpret_cast<int32_t*>(at(workspace, w.counts));
  int32_t* dropped = num_dropped ? num_dropped : reinterpret_cast<int32_t*>(at(workspace, w.dropped));
  int32_t* offsets = reinterpret_cast<int32_t*>(at(workspace, w.offsets));
  int32_t* perm_src = reinterpret_cast<int32_t*>(at(workspace, w.perm_src));
  int32_t* slot_pos = reinterpret_cast<int32_t*>(at(workspace, w.slot_pos));
  void* eout = at(workspace, w.eout);
  void* sout = cfg->num_shared > 0 ? at(workspace, w.sout) : nullptr;
  // the permutation also writes the GEMM tile plans when it runs as one
  // workgroup (small batches), which saves the plan kernel's launch
  const FfnPasses passes = ffn_passes(cfg, T, x, nullptr, perm_src, offsets, w1, w3, w2, ws1,
                                      ws3, ws2, eout, sout, at(workspace, w.ffn));
  PlanSpec spec{};
  const bool have_spec = ffn_plan_spec(passes.p, passes.p2, &spec);
  bool built = false;
  const RouteArgs ra = route_args(cfg, T, x, w_router, logit_offset, select_bias, nullptr, idx,
                                  gate, route_ws_bytes(T, cfg->num_experts, cfg->dtype)
                                            ? at(workspace, w.route) : nullptr);
  const PermuteArgs pa = permute_args(cfg, T, idx, x, counts, offsets, perm_src, slot_pos,
                                      dropped, nullptr, at(workspace, w.perm),
                                      have_spec ? &spec : nullptr);
  if (route_permute_small_ok(ra, pa)) {
    // decode batches: router and permutation in two launches instead of three
    st = hip_status(launch_route_permute_small(ra, pa, s, &built));
    if (st != MOE_OK) return st;
  } else {
    st = hip_status(launch_route(ra, s));
    if (st != MOE_OK) return st;
    st = hip_status(launch_permute(pa, s, &built));
    if (st != MOE_OK) return st;
  }
  st = run_ffn(passes, built, s);
  if (st != MOE_OK) return st;
  return do_combine(cfg, T, eout, slot_pos, gate, sout, y, s);
}

}  // namespace

extern "C" {

const char* moe_status_str(moe_status_t st) {
  switch (st) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG: invalid argument";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED: configuration not supported";
    case MOE_ERR_WORKSPACE:
      return "MOE_ERR_WORKSPACE: workspace too small (or, for moe_forward_noalloc, the batch's "
             "workspace exceeds MOE_NOALLOC_SCRATCH_BYTES)";
    case MOE_ERR_HIP: return "MOE_ERR_HIP: HIP runtime or launch error";
  }
  return "unknown moe_status_t";
}

moe_status_t moe_check_config(const moe_config_t* cfg, int64_t T) { return check_cfg(cfg, T); }

moe_status_t moe_workspace_size(const moe_config_t* cfg, int64_t T, size_t* bytes) {
  moe_status_t st = check_cfg(cfg, T);
  if (st != MOE_OK) return st;
  if (!bytes) return MOE_ERR_INVALID_ARG;
  *bytes = fwd_ws(cfg, T).total;
  return MOE_OK;
}

moe_status_t moe_capacity(const moe_config_t* cfg, int64_t T, int64_t* capacity) {
  moe_status_t st = check_cfg(cfg, T);
  if (st != MOE_OK) return st;
  if (!capacity) return MOE_ERR_INVALID_ARG;
  *capacity = capacity_of(cfg, T);
  return MOE_OK;
}

moe_status_t moe_route(const moe_config_t* cfg, int64_t T, const void* x, const void* w_router,
                       const float* logit_offset, const float* select_bias, float* logits,
                       int32_t* topk_idx, float* topk_gate, void* workspace, size_t ws_bytes,
                       void* stream) {
  moe_status_t st = check_cfg(cfg, T);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;  // nothing to do; token-sized pointers may be null
  if (!x || !w_router || !topk_idx || !topk_gate) return MOE_ERR_INVALID_ARG;
  if (!al(x, 16) || !al(w_router, 16) || !al(topk_idx, 4) || !al(topk_gate, 4) ||
      (logits && !al(logits, 4)) || (logit_offset && !al(logit_offset, 4)) ||
      (select_bias && !al(select_bias, 4)))
    return MOE_ERR_INVALID_ARG;
  if (workspace && !al(workspace, ALIGN)) return MOE_ERR_INVALID_ARG;
  const size_t need = route_ws_bytes(T, cfg->num_experts, cfg->dtype);
  void* part = (workspace && ws_bytes >= need && need > 0) ? workspace : nullptr;
  return do_route(cfg, T, x, w_router, logit_offset, select_bias, logits, topk_idx, topk_gate,
                  part, static_cast<hipStream_t>(stream));
}

moe_status_t moe_permute(const moe_config_t* cfg, int64_t T, const int32_t* topk_idx,
                         const void* x, int32_t* expert_counts, int32_t* expert_offsets,
                         int32_t* perm_src, int32_t* slot_pos, int32_t* num_dropped,
                         void* x_perm, void* workspace, size_t ws_bytes, void* stream) {
  moe_status_t st = check_cfg(cfg, T);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;  // nothing to do; token-sized pointers may be null
  if (!topk_idx || !expert_offsets || !perm_src || !slot_pos) return MOE_ERR_INVALID_ARG;
  if (x_perm && (!x || !al(x, 16) || !al(x_perm, 16))) return MOE_ERR_INVALID_ARG;
  if (!al(topk_idx, 4) || !al(expert_offsets, 4) || !al(perm_src, 4) || !al(slot_pos, 4) ||
      (expert_counts && !al(expert_counts, 4)) || (num_dropped && !al(num_dropped, 4)))
    return MOE_ERR_INVALID_ARG;
  if (!workspace || !al(workspace, ALIGN)) return MOE_ERR_INVALID_ARG;
  if (ws_bytes < fwd_ws(cfg, T).total) return MOE_ERR_WORKSPACE;
  return do_permute(cfg, T, topk_idx, x, expert_counts, expert_offsets, perm_src, slot_pos,
                    num_dropped, x_perm, workspace, static_cast<hipStream_t>(stream));
}

moe_status_t moe_expert_ffn(const moe_config_t* cfg, int64_t T, const void* x,
                            const void* x_perm, const int32_t* expert_offsets, const void* w1,
                            const void* w3, const void* w2, const void* ws1, const void* ws3,
                            const void* ws2, void* expert_out, void* shared_out,
                            void* workspace, size_t ws_bytes, void* stream) {
  moe_status_t st = check_cfg(cfg, T);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;  // nothing to do; token-sized pointers may be null
  if (!x_perm || !expert_offsets || !w1 || !w2 || !expert_out) return MOE_ERR_INVALID_ARG;
  if (cfg->act == MOE_ACT_SWIGLU && !w3) return MOE_ERR_INVALID_ARG;
  if (cfg->num_shared > 0 && (!x || !ws1 || !ws3 || !ws2 || !shared_out))
    return MOE_ERR_INVALID_ARG;
  const void* p16[] = {x_perm, w1, w2, expert_out, w3, x, ws1, ws3, ws2, shared_out};
  for (const void* p : p16)
    if (p && !al(p, 16)) return MOE_ERR_INVALID_ARG;
  if (!al(expert_offsets, 4)) return MOE_ERR_INVALID_ARG;
  if (!workspace || !al(workspace, ALIGN)) return MOE_ERR_INVALID_ARG;
  if (ws_bytes < fwd_ws(cfg, T).total) return MOE_ERR_WORKSPACE;
  return do_ffn(cfg, T, x, x_perm, nullptr, expert_offsets, w1, w3, w2, ws1, ws3, ws2,
                expert_out, shared_out, workspace, static_cast<hipStream_t>(stream));
}

moe_status_t moe_combine(const moe_config_t* cfg, int64_t T, const void* expert_out,
                         const int32_t* slot_pos, const float* topk_gate, const void* shared_out,
                         void* y, void* stream) {
  moe_status_t st = check_cfg(cfg, T);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;  // nothing to do; token-sized pointers may be null
  if (!expert_out || !slot_pos || !topk_gate || !y) return MOE_ERR_INVALID_ARG;
  if (!al(expert_out, 16) || !al(y, 16) || (shared_out && !al(shared_out, 16)) ||
      !al(slot_pos, 4) || !al(topk_gate, 4))
    return MOE_ERR_INVALID_ARG;
  return do_combine(cfg, T, expert_out, slot_pos, topk_gate, shared_out, y,
                    static_cast<hipStream_t>(stream));
}

moe_status_t moe_forward(const moe_config_t* cfg, int64_t T, const void* x, const void* w_router,
                         const float* logit_offset, const float* select_bias, const void* w1,
                         const void* w3, const void* w2, const void* ws1, const void* ws3,
                         const void* ws2, void* y, int32_t* topk_idx, float* topk_gate,
                         int32_t* expert_counts, int32_t* num_dropped, void* workspace,
                         size_t ws_bytes, void* stream) {
  return forward_impl(cfg, T, x, w_router, logit_offset, select_bias, w1, w3, w2, ws1, ws3, ws2,
                      y, topk_idx, topk_gate, expert_counts, num_dropped, workspace, ws_bytes,
                      stream, false);
}

moe_status_t moe_forward_noalloc(const moe_config_t* cfg, int64_t T, const void* x,
                                 const void* w_router, const float* logit_offset,
                                 const float* select_bias, const void* w1, const void* w3,
                                 const void* w2, const void* ws1, const void* ws3,
                                 const void* ws2, void* y, int32_t* topk_idx, float* topk_gate,
                                 int32_t* expert_counts, int32_t* num_dropped, void* stream) {
  return forward_impl(cfg, T, x, w_router, logit_offset, select_bias, w1, w3, w2, ws1, ws3, ws2,
                      y, topk_idx, topk_gate, expert_counts, num_dropped, nullptr, 0, stream,
                      true);
}

moe_status_t moe_profile_enable(int32_t on) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  for (auto& r : g_prof_recs) {
    g_prof_pool.push_back(r.e0);
    g_prof_pool.push_back(r.e1);
  }
  g_prof_recs.clear();
  ++g_prof_gen;
  g_prof_on.store(on != 0, std::memory_order_relaxed);
  return MOE_OK;
}

int32_t moe_profile_read(const char** names, double* total_ms, int32_t* launches,
                         int32_t max_names) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  std::vector<const char*> nm;
  std::vector<double> tot;
  std::vector<int32_t> cnt;
  int32_t rc = 0;
  for (auto& r : g_prof_recs) {
    float ms = 0.f;
    if (hipEventSynchronize(r.e1) != hipSuccess || hipEventElapsedTime(&ms, r.e0, r.e1) != hipSuccess) {
      rc = -1;
      continue;
    }
    size_t i = 0;
    for (; i < nm.size(); ++i)
      if (strcmp(nm[i], r.name) == 0) break;
    if (i == nm.size()) {
      nm.push_back(r.name);
      tot.push_back(0.0);
      cnt.push_back(0);
    }
    tot[i] += ms;
    cnt[i] += 1;
  }
  for (auto& r : g_prof_recs) {
    g_prof_pool.push_back(r.e0);
    g_prof_pool.push_back(r.e1);
  }
  g_prof_recs.clear();
  ++g_prof_gen;
  if (rc < 0) return -1;
  int32_t n = 0;
  for (size_t i = 0; i < nm.size() && n < max_names; ++i, ++n) {
    if (names) names[n] = nm[i];
    if (total_ms) total_ms[n] = tot[i];
    if (launches) launches[n] = cnt[i];
  }
  return n;
}

moe_status_t moe_routing_stats(const moe_config_t* cfg, int64_t T, const float* logits,
                               const int32_t* expert_counts, const int32_t* num_dropped,
                               const float* select_bias, float gamma, float alpha, float* f,
                               float* P, float* loss, float* drop_rate, float* bias_out,
                               void* workspace, size_t ws_bytes, void* stream) {
  moe_status_t st = check_cfg(cfg, T);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  if (!logits || !expert_counts || !f || !P || !loss) return MOE_ERR_INVALID_ARG;
  if (drop_rate && !num_dropped) return MOE_ERR_INVALID_ARG;
  if (bias_out && !select_bias) return MOE_ERR_INVALID_ARG;
  if (!(gamma >= 0.f) || !(alpha >= 0.f)) return MOE_ERR_INVALID_ARG;   // also rejects NaN
  if (!al(logits, 4) || !al(expert_counts, 4) || !al(f, 4) || !al(P, 4) || !al(loss, 4) ||
      (num_dropped && !al(num_dropped, 4)) || (select_bias && !al(select_bias, 4)) ||
      (drop_rate && !al(drop_rate, 4)) || (bias_out && !al(bias_out, 4)))
    return MOE_ERR_INVALID_ARG;
  if (workspace && !al(workspace, ALIGN)) return MOE_ERR_INVALID_ARG;
  const FwdWs w = fwd_ws(cfg, T);
  if (!workspace || ws_bytes < w.total) return MOE_ERR_WORKSPACE;
  StatsArgs a;
  a.logits = logits;
  a.counts = expert_counts;
  a.dropped = num_dropped;
  a.bias = select_bias;
  a.gamma = gamma;
  a.alpha = alpha;
  a.f = f;
  a.P = P;
  a.loss = loss;
  a.drop_rate = drop_rate;
  a.bias_out = bias_out;
  a.partial = reinterpret_cast<float*>(at(workspace, w.stats));
  a.T = T;
  a.E = cfg->num_experts;
  a.k = cfg->top_k;
  return hip_status(launch_stats(a, static_cast<hipStream_t>(stream)));
}


moe_status_t moe_train_workspace_size(const moe_config_t* cfg, int64_t T, size_t* bytes) {
  moe_status_t st = check_cfg(cfg, T);
  if (st != MOE_OK) return st;
  if (!bytes) return MOE_ERR_INVALID_ARG;
  if (cfg->dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  *bytes = train_ws(cfg, T).total;
  return MOE_OK;
}

moe_status_t moe_forward_train(const moe_config_t* cfg, int64_t T, const void* x,
                               const void* w_router, const float* logit_offset,
                               const float* select_bias, const void* w1, const void* w3,
                               const void* w2, const void* ws1, const void* ws3, const void* ws2,
                               void* y, void* saved, size_t saved_bytes, void* stream) {
  moe_status_t st = check_cfg(cfg, T);
  if (st != MOE_OK) return st;
  if (cfg->dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!x || !w_router || !w1 || !w2 || !y) return MOE_ERR_INVALID_ARG;
  if (cfg->act == MOE_ACT_SWIGLU && !w3) return MOE_ERR_INVALID_ARG;
  if (cfg->num_shared > 0 && (!ws1 || !ws3 || !ws2)) return MOE_ERR_INVALID_ARG;
  const void* p16[] = {x, w_router, w1, w2, y, w3, ws1, ws3, ws2};
  for (const void* p : p16)
    if (p && !al(p, 16)) return MOE_ERR_INVALID_ARG;
  if ((logit_offset && !al(logit_offset, 4)) || (select_bias && !al(select_bias, 4)))
    return MOE_ERR_INVALID_ARG;
  if (!saved || !al(saved, ALIGN)) return MOE_ERR_INVALID_ARG;
  const TrainWs tw = train_ws(cfg, T);
  if (saved_bytes < tw.total) return MOE_ERR_WORKSPACE;
  const FwdWs& w = tw.fwd;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int32_t* idx = reinterpret_cast<int32_t*>(at(saved, w.idx));
  float* gate = reinterpret_cast<float*>(at(saved, w.gate));
  int32_t* counts = reinterpret_cast<int32_t*>(at(saved, w.counts));
  int32_t* dropped = reinterpret_cast<int32_t*>(at(saved, w.dropped));
  int32_t* offsets = reinterpret_cast<int32_t*>(at(saved, w.offsets));
  int32_t* perm_src = reinterpret_cast<int32_t*>(at(saved, w.perm_src));
  int32_t* slot_pos = reinterpret_cast<int32_t*>(at(saved, w.slot_pos));
  float* logits = reinterpret_cast<float*>(at(saved, tw.logits));
  void* x_perm = at(saved, tw.x_perm);
  void* eout = at(saved, w.eout);
  void* sout = cfg->num_shared > 0 ? at(saved, w.sout) : nullptr;
  st = do_route(cfg, T, x, w_router, logit_offset, select_bias, logits, idx, gate,
                route_ws_bytes(T, cfg->num_experts, cfg->dtype) ? at(saved, w.route) : nullptr, s);
  if (st != MOE_OK) return st;
  // the rows are gathered once (the weight gradients read them again)
  const FfnPasses passes = ffn_passes(cfg, T, x, x_perm, perm_src, offsets, w1, w3, w2, ws1, ws3,
                                      ws2, eout, sout, at(saved, w.ffn), &tw, saved);
  PlanSpec spec{};
  const bool have_spec = ffn_plan_spec(passes.p, passes.p2, &spec);
  bool built = false;
  st = do_permute(cfg, T, idx, x, counts, offsets, perm_src, slot_pos, dropped, x_perm,
                  at(saved, w.perm), s, have_spec ? &spec : nullptr, &built);
  if (st != MOE_OK) return st;
  st = run_ffn(passes, built, s);
  if (st != MOE_OK) return st;
  return do_combine(cfg, T, eout, slot_pos, gate, sout, y, s);
}

moe_status_t moe_saved_routing(const moe_config_t* cfg, int64_t T, void* saved,
                               float** logits, int32_t** topk_idx, float** topk_gate,
                               int32_t** expert_counts, int32_t** num_dropped,
                               int32_t** expert_offsets, int32_t** slot_pos) {
  moe_status_t st = check_cfg(cfg, T);
  if (st != MOE_OK) return st;
  if (cfg->dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (!saved) return MOE_ERR_INVALID_ARG;
  const TrainWs tw = train_ws(cfg, T);
  if (logits) *logits = reinterpret_cast<float*>(at(saved, tw.logits));
  if (topk_idx) *topk_idx = reinterpret_cast<int32_t*>(at(saved, tw.fwd.idx));
  if (topk_gate) *topk_gate = reinterpret_cast<float*>(at(saved, tw.fwd.gate));
  if (expert_counts) *expert_counts = reinterpret_cast<int32_t*>(at(saved, tw.fwd.counts));
  if (num_dropped) *num_dropped = reinterpret_cast<int32_t*>(at(saved, tw.fwd.dropped));
  if (expert_offsets) *expert_offsets = reinterpret_cast<int32_t*>(at(saved, tw.fwd.offsets));
  if (slot_pos) *slot_pos = reinterpret_cast<int32_t*>(at(saved, tw.fwd.slot_pos));
  return MOE_OK;
}

moe_status_t moe_backward_workspace_size(const moe_config_t* cfg, int64_t T, size_t* bytes) {
  moe_status_t st = check_cfg(cfg, T);
  if (st != MOE_OK) return st;
  if (!bytes) return MOE_ERR_INVALID_ARG;
  if (cfg->dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  *bytes = bwd_ws(cfg, T).total;
  return MOE_OK;
}

moe_status_t moe_backward(const moe_config_t* cfg, int64_t T, const void* x, const void* w_router,
                          const void* w1, const void* w3, const void* w2, const void* ws1,
                          const void* ws3, const void* ws2, const void* saved, size_t saved_bytes,
                          const void* dy, float aux_alpha, void* dx, float* dw_router, void* dw1,
                          void* dw3, void* dw2, void* dws1, void* dws3, void* dws2,
                          float* d_gate, float* d_logits, void* workspace, size_t ws_bytes,
                          void* stream) {
  moe_status_t st = check_cfg(cfg, T);
  if (st != MOE_OK) return st;
  if (cfg->dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (!(aux_alpha >= 0.f) || isinf(aux_alpha)) return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;
  const bool glu = cfg->act == MOE_ACT_SWIGLU;
  const int S = cfg->num_shared;
  if (!x || !w_router || !w1 || !w2 || !saved || !dy || !dx || !dw_router || !dw1 || !dw2)
    return MOE_ERR_INVALID_ARG;
  if (glu && (!w3 || !dw3)) return MOE_ERR_INVALID_ARG;
  if (S > 0 && (!ws1 || !ws3 || !ws2 || !dws1 || !dws3 || !dws2)) return MOE_ERR_INVALID_ARG;
  const void* p16[] = {x, w_router, w1, w2, w3, ws1, ws3, ws2, dy, dx, dw_router, dw1, dw3, dw2,
                       dws1, dws3, dws2};
  for (const void* p : p16)
    if (p && !al(p, 16)) return MOE_ERR_INVALID_ARG;
  if ((d_gate && !al(d_gate, 4)) || (d_logits && !al(d_logits, 4))) return MOE_ERR_INVALID_ARG;
  if (!al(saved, ALIGN) || !workspace || !al(workspace, ALIGN)) return MOE_ERR_INVALID_ARG;
  const TrainWs tw = train_ws(cfg, T);
  const BwdWs bw = bwd_ws(cfg, T);
  if (saved_bytes < tw.total || ws_bytes < bw.total) return MOE_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t R = T * cfg->top_k;
  const int E = cfg->num_experts, d = cfg->d, dff = cfg->d_ff, dffs = cfg->d_ff_shared;
  const FwdWs& fw = tw.fwd;
  const FfnWs ffw = ffn_ws(cfg, T);
  const char* fbase = at(saved, fw.ffn);
  const int32_t* offsets = reinterpret_cast<const int32_t*>(at(saved, fw.offsets));
  const int32_t* slot_pos = reinterpret_cast<const int32_t*>(at(saved, fw.slot_pos));
  const int32_t* idx = reinterpret_cast<const int32_t*>(at(saved, fw.idx));
  float* dlog = d_logits ? d_logits : reinterpret_cast<float*>(at(workspace, bw.dlogits));
  void* zero = at(workspace, bw.zero);
  void* dO = at(workspace, bw.dO);
  void* dG = at(workspace, bw.dG);
  void* dU = glu ? at(workspace, bw.dU) : nullptr;
  void* dXp = at(workspace, bw.dXp);
  if (launch_zero(zero, kZeroBytes, s) != hipSuccess) return MOE_ERR_HIP;

  // gates: dO, dg, ds
  GateBwdArgs ga;
  memset(&ga, 0, sizeof(ga));
  ga.dy = static_cast<const uint16_t*>(dy);
  ga.eout = reinterpret_cast<const uint16_t*>(at(saved, fw.eout));
  ga.slot_pos = slot_pos;
  ga.topk_idx = idx;
  ga.gate = reinterpret_cast<const float*>(at(saved, fw.gate));
  ga.logits = reinterpret_cast<const float*>(at(saved, tw.logits));
  ga.counts = reinterpret_cast<const int32_t*>(at(saved, fw.counts));
  ga.aux_scale = (float)((double)aux_alpha * E / ((double)T * (double)T));
  ga.d_out = static_cast<uint16_t*>(dO);
  ga.d_gate = d_gate;
  ga.d_logits = dlog;
  ga.T = T;
  ga.d = d;
  ga.k = cfg->top_k;
  ga.E = E;
  ga.gating = cfg->gating;
  if (launch_gate_bwd(ga, s) != hipSuccess) return MOE_ERR_HIP;

  const int epi = glu ? 3 : (cfg->act == MOE_ACT_GELU ? 2 : 1);
  auto run_expert_grads = [&](bool shared) -> moe_status_t {
    // one set of experts: routed (segments = expert rows) or shared (dense)
    const int G = shared ? S : E;
    const int64_t rows = shared ? (int64_t)S * T : R;
    const int f = shared ? dffs : dff;
    const int32_t* seg = shared ? nullptr : offsets;
    void* plan_h = at(workspace, shared ? bw.splan_h : bw.plan_h);
    void* plan_x = at(workspace, shared ? bw.splan_x : bw.plan_x);
    PlanSpec ps{};
    ps.balanced = 0;   // the backward GEMMs store full row tiles through LDS
    ps.BM = bwd_tile_rows();
    ps.NT = (f + bwd_tile_cols() - 1) / bwd_tile_cols();
    ps.NT2 = (d + bwd_tile_cols() - 1) / bwd_tile_cols();
    const int split = shared ? 1 : bw.split;
    ps.S2 = 1;
    if (split > 1) {   // the dX plan lists the tail tiles' K parts after the whole tiles
      const int cus = cu_count();
      ps.tail_cus = cus < kTailParts ? cus : kTailParts;
    }
    ps.plan = static_cast<int32_t*>(plan_h);
    ps.plan2 = static_cast<int32_t*>(plan_x);
    if (launch_plan_kernel(seg, G, T, ps, s) != hipSuccess) return MOE_ERR_HIP;
    const void* Gsv = shared ? at(saved, tw.ssave1) : at(saved, tw.save1);
    const void* Usv = shared ? at(saved, tw.ssave2) : (glu ? at(saved, tw.save2) : nullptr);
    const void* Hin = shared ? fbase + ffw.Hs : fbase + ffw.H;
    void* gG = shared ? at(workspace, bw.dGs) : dG;
    void* gU = shared ? at(workspace, bw.dUs) : dU;
    void* gX = shared ? at(workspace, bw.dXs) : dXp;
    const void* gO = shared ? dy : dO;
    const void* Xin = shared ? x : at(saved, tw.x_perm);
    const int e1 = shared ? 3 : epi;
    const bool g2 = shared || glu;
    BwdGemm b;
    // dH = dO . W2 -> dG, dU (or dZ)
    memset(&b, 0, sizeof(b));
    b.kind = BG_DH;
    b.epi = e1;
    b.name = shared ? "bwd_dh_shared" : "bwd_dh";
    b.P = shared ? ws2 : w2;
    b.ldp = f;
    b.p_seg = (int64_t)d * f;
    b.Q = gO;
    b.ldq = d;
    b.q_row_seg = 0;
    b.C = gG;
    b.C2 = gU;
    b.ldc = f;
    b.c_row_seg = shared ? T : 0;
    b.S1 = Gsv;
    b.S2 = Usv;
    b.plan = plan_h;
    b.max_entries = bwd_entries(rows, G, f);
    b.K = d;
    b.N = f;
    b.G = G;
    if (launch_bwd_gemm(b, s) != hipSuccess) return MOE_ERR_HIP;
    // dW2 = dO^T H
    memset(&b, 0, sizeof(b));
    b.kind = BG_DW;
    b.name = shared ? "bwd_dw2_shared" : "bwd_dw2";
    b.P = Hin;
    b.ldp = f;
    b.p_row_seg = shared ? T : 0;
    b.Q = gO;
    b.ldq = d;
    b.q_row_seg = 0;
    b.C = shared ? dws2 : dw2;
    b.ldc = f;
    b.c_seg = (int64_t)d * f;
    b.seg = seg;
    b.order = reinterpret_cast<int32_t*>(at(workspace, bw.order));
    b.dense_rows = T;
    b.zero = zero;
    b.M = d;
    b.N = f;
    b.G = G;
    if (launch_bwd_gemm(b, s) != hipSuccess) return MOE_ERR_HIP;
    // dX = dG . W1 (+ dU . W3)
    memset(&b, 0, sizeof(b));
    b.kind = BG_DX;
    b.epi = g2 ? 1 : 0;
    b.name = shared ? "bwd_dx_shared" : "bwd_dx";
    b.P = shared ? ws1 : w1;
    b.P2 = g2 ? (shared ? ws3 : w3) : nullptr;
    b.ldp = d;
    b.p_seg = (int64_t)f * d;
    b.Q = gG;
    b.Q2 = g2 ? gU : nullptr;
    b.ldq = f;
    b.q_row_seg = shared ? T : 0;
    b.C = gX;
    b.ldc = d;
    b.c_row_seg = shared ? T : 0;
    b.plan = plan_x;
    b.max_entries = bwd_entries(rows, G, d) + (split > 1 ? kTailParts : 0);
    b.K = f;
    b.N = d;
    b.G = G;
    b.part = split > 1 ? reinterpret_cast<float*>(at(workspace, bw.dXpart)) : nullptr;
    if (launch_bwd_gemm(b, s) != hipSuccess) return MOE_ERR_HIP;
    if (split > 1 &&
        launch_tail_reduce(plan_x, b.part, gX, d, 0, "bwd_dx_tail_reduce", s) != hipSuccess)
      return MOE_ERR_HIP;
    // dW1 = dG^T X, dW3 = dU^T X
    for (int u = 0; u < (g2 ? 2 : 1); ++u) {
      memset(&b, 0, sizeof(b));
      b.kind = BG_DW;
      b.name = shared ? (u ? "bwd_dw3_shared" : "bwd_dw1_shared") : (u ? "bwd_dw3" : "bwd_dw1");
      b.P = Xin;
      b.ldp = d;
      b.p_row_seg = 0;
      b.Q = u ? gU : gG;
      b.ldq = f;
      b.q_row_seg = shared ? T : 0;
      b.C = shared ? (u ? dws3 : dws1) : (u ? dw3 : dw1);
      b.ldc = d;
      b.c_seg = (int64_t)f * d;
      b.seg = seg;
      b.order = reinterpret_cast<int32_t*>(at(workspace, bw.order));
      b.dense_rows = T;
      b.zero = zero;
      b.M = f;
      b.N = d;
      b.G = G;
      if (launch_bwd_gemm(b, s) != hipSuccess) return MOE_ERR_HIP;
    }
    return MOE_OK;
  };
  st = run_expert_grads(false);
  if (st != MOE_OK) return st;
  if (S > 0) {
    st = run_expert_grads(true);
    if (st != MOE_OK) return st;
  }

  DxArgs xa;
  xa.dxp = static_cast<const uint16_t*>(dXp);
  xa.dxs = S > 0 ? reinterpret_cast<const uint16_t*>(at(workspace, bw.dXs)) : nullptr;
  xa.slot_pos = slot_pos;
  xa.topk_idx = idx;
  xa.d_logits = dlog;
  xa.w_router = static_cast<const uint16_t*>(w_router);
  xa.dx = static_cast<uint16_t*>(dx);
  xa.T = T;
  xa.d = d;
  xa.k = cfg->top_k;
  xa.E = E;
  xa.S = S;
  xa.sparse_ds = cfg->gating != MOE_GATE_SOFTMAX_FULL && aux_alpha == 0.f;
  if (launch_dx(xa, s) != hipSuccess) return MOE_ERR_HIP;

  WrArgs wa;
  wa.d_logits = dlog;
  wa.x = static_cast<const uint16_t*>(x);
  wa.dw_router = dw_router;
  wa.partial = reinterpret_cast<float*>(at(workspace, bw.wr));
  wa.T = T;
  wa.E = E;
  wa.d = d;
  wa.chunk = 0;
  return hip_status(launch_router_bwd(wa, s));
}

}  // extern "C"
