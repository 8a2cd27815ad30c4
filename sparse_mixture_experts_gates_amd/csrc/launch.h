// Internal launcher API between the C-ABI host code (moe_api.hip) and the
// kernel files.  Every launcher enqueues on `stream` and returns the result of
// hipGetLastError() after its launches.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// Named-kernel launch bracket for the optional event profiler (moe_api.hip):
// prof_before records the start event and returns a handle (-1 when the
// profiler is off) that the matching prof_after takes, so launches from
// several host threads pair their own events.
int64_t prof_before(const char* name, hipStream_t s);
void prof_after(int64_t rec, hipStream_t s);

// Compute units of the current device (one persistent workgroup each).
int cu_count();

struct RouteArgs {
  const void* x;
  const void* w;
  const float* offset;  // [E] or null
  const float* bias;    // [E] or null
  float* logits;        // [T, E] or null
  int32_t* topk_idx;    // [T, k]
  float* topk_gate;     // [T, k]
  float* partial;       // optional workspace for the split-K small-batch path
  int64_t T;
  int d, E, k, gating, dtype;
};
size_t route_ws_bytes(int64_t T, int E, int dtype);
hipError_t launch_route(const RouteArgs& a, hipStream_t s);

// Where and how the tile plans of an expert FFN's two GEMM passes go (same
// row tiling): row tile height, column tiles per pass, and the two plan
// buffers (header + entries).
struct PlanSpec {
  int BM, NT, NT2;
  int S2;                   // K parts of the second pass (1 = not split)
  int32_t* plan;
  int32_t* plan2;
  int balanced;             // 1: a segment's rows split into equal row tiles
                            // (multiples of 16 rows, at most BM); 0: tiles of
                            // BM rows and one ragged last tile
  int tail_cus;             // > 0: the second pass (S2 = 1) lists its whole
                            // tiles for the per-XCD queues, and the tiles of a
                            // partial last round over tail_cus CUs in K parts
                            // (a shared tail queue); 0: no tail split
};
// Tail split of a second expert GEMM: at most this many K-part entries (and
// fp32 partial tiles of 256 x 256 in the workspace).
constexpr int kTailParts = 256;
constexpr int kTailMaxSplit = 8;

struct PermuteArgs {
  const int32_t* topk_idx;  // [T*k]
  const void* x;            // [T, d] (may be null when x_perm is null)
  int32_t* counts;          // [E] or null
  int32_t* offsets;         // [E+1]
  int32_t* perm_src;        // [T*k]
  int32_t* slot_pos;        // [T*k]
  int32_t* num_dropped;     // [1] or null
  void* x_perm;             // [T*k, d] or null
  int32_t* block_counts;    // workspace [nblocks * E]
  int32_t* kept_total;      // workspace [1]: expert_offsets[E] copy for the gather
  int64_t T;
  int k, E, d, dtype;
  int64_t capacity;         // < 0: unlimited
  int slot_major;           // capacity and row order by slot, then token
  const PlanSpec* plans;    // optional: the routed experts' GEMM plans, built
                            // here when the one-workgroup path runs
};
int permute_nblocks(int64_t rows);
// Small batches (bf16, 1 <= T <= 16, router workspace given, no x_perm): the
// router's score parts, then one workgroup that adds them, selects the top-k
// and runs the whole permutation (plans included when pa.plans is set).
bool route_permute_small_ok(const RouteArgs& ra, const PermuteArgs& pa);
hipError_t launch_route_permute_small(const RouteArgs& ra, const PermuteArgs& pa, hipStream_t s,
                                      bool* plans_built);
// *plans_built (if given) tells whether a.plans were written.
hipError_t launch_permute(const PermuteArgs& a, hipStream_t s, bool* plans_built = nullptr);

// One grouped GEMM pass over ragged row segments:
//   C[r, n] = epilogue( sum_k A[r, k] * W_seg[n, k] )  for r in the segment.
// mode: 0 = plain, 1 = relu, 2 = gelu, 3 = swiglu (W1 = w, W3 = w_up).
struct FfnPassArgs {
  const void* A;          // [rows, K] dtype, or [T, K] read through a_rows
  const int32_t* a_rows;  // optional: A row of permuted row p is a_rows[p] / a_div
  int a_div;
  const void* w;          // [G, N_w, K] dtype (gate / only matrix)
  const void* w_up;       // [G, N_w, K] dtype (SwiGLU up) or null
  void* C;                // [rows, N] dtype
  const int32_t* seg_offsets;  // [G+1] device row offsets, or null = one dense segment
  int64_t dense_rows;     // rows when seg_offsets is null
  int G;                  // number of segments (experts)
  int K, N;               // N = output columns (d_ff for GEMM1, d for GEMM2)
  int mode, dtype;
  int64_t a_seg_rows;     // row offset of segment g in A is g * a_seg_rows (dense segments)
  int64_t c_seg_rows;     // row offset of segment g in C is g * c_seg_rows
  void* plan;             // workspace for the tile plan
  int64_t max_rows;       // upper bound of rows over all segments (host)
  bool small;             // small-batch (decode) tile shape
  int split;              // second GEMM only: > 1 = the partial last round of
                          // tiles runs in K parts (see PlanSpec::tail_cus)
  float* part;            // split: fp32 partial tiles [kTailParts][256][256]
  // first GEMM, training forward: the pre-activations in dtype, laid out like
  // C -- SwiGLU: W1 x to save1 and W3 x to save2; ReLU / GeLU: W1 x to save1
  void* save1;
  void* save2;
};
size_t ffn_plan_bytes(int64_t max_rows, int G, int N, bool small, int dtype, int split = 1);
// Plans of two passes with the same row tiles (ps.BM) over G segments (row
// offsets seg[G+1], or G dense segments of dense_rows rows).
hipError_t launch_plan_kernel(const int32_t* seg, int G, int64_t dense_rows, const PlanSpec& ps,
                              hipStream_t s);
// 2 when a routed second GEMM pass of this shape splits the tiles of its
// partial last round over K (decided on the device from the real tile
// count), else 1.
int ffn_split(int64_t max_rows, int G, int N, int K, bool small, int dtype);
// For a split pass: C = bf16(sum of the K parts, in order) on the tail tiles.
hipError_t launch_ffn_tail_reduce(const FfnPassArgs& p, hipStream_t s);
// The same for any pass on 256 x 256 tiles whose plan (header + entries) has
// a tail split: C[g * c_seg_rows + row, col] with row pitch N, from the fp32
// partial tiles part[kTailParts][256][256].
hipError_t launch_tail_reduce(const void* plan, const float* part, void* C, int N,
                              int64_t c_seg_rows, const char* name, hipStream_t s);
// The plan layout of the two passes of one expert FFN; false if there is
// nothing to plan (no rows).
bool ffn_plan_spec(const FfnPassArgs& p1, const FfnPassArgs& p2, PlanSpec* ps);
// One plan kernel for the two passes of an expert FFN (same row tiles; the
// entries go to p1.plan and p2.plan), then one GEMM launch per pass.
hipError_t launch_ffn_plans(const FfnPassArgs& p1, const FfnPassArgs& p2, hipStream_t s);
hipError_t launch_ffn_pass(const FfnPassArgs& a, hipStream_t s);

// Routing statistics (balance signals) of one batch.
struct StatsArgs {
  const float* logits;      // [T, E] router scores
  const int32_t* counts;    // [E] assignments per expert before capacity
  const int32_t* dropped;   // [1] (read only when drop_rate is set)
  const float* bias;        // [E] (read only when bias_out is set)
  float gamma, alpha;
  float* f;                 // [E]
  float* P;                 // [E]
  float* loss;              // [1]
  float* drop_rate;         // [1] or null
  float* bias_out;          // [E] or null (may alias bias)
  float* partial;           // workspace, stats_ws_bytes()
  int64_t T;
  int E, k;
};
int stats_nblocks(int64_t T);
size_t stats_ws_bytes(int64_t T, int E);
hipError_t launch_stats(const StatsArgs& a, hipStream_t s);

struct CombineArgs {
  const void* expert_out;   // [T*k, d]
  const int32_t* slot_pos;  // [T*k]
  const float* gate;        // [T*k]
  const void* shared_out;   // [S, T, d] or null
  void* y;                  // [T, d]
  int64_t T;
  int k, d, S, dtype;
};
hipError_t launch_combine(const CombineArgs& a, hipStream_t s);

// ------------------------------------------------------------ backward pass
// Backward grouped GEMMs (bf16).  Output C[m, n] = sum_k P(n, k) Q(m, k):
//  BG_DH  rows m of each expert's segment (plan), P = weights W2_e read as
//         (n = d_ff column, k = d row), Q = dO rows (k contiguous); epilogue
//         epi 0 plain, 1 ReLU', 2 GeLU', 3 SwiGLU (C = dG, C2 = dU from the
//         saved S1 = W1 x, S2 = W3 x)
//  BG_DX  rows m (plan), P = W1_e (+ W3_e as P2) read as (n = d column, k =
//         d_ff row), Q = dG (+ dU as Q2); epi 1 = two operand pairs
//  BG_DW  per segment g a full M x N output, k over the segment's rows:
//         P(n, k) = P[(g p_row_seg + r0 + k) ldp + n], Q(m, k) likewise
enum { BG_DH = 0, BG_DX = 1, BG_DW = 2 };
struct BwdGemm {
  int kind, epi;
  const char* name;
  const void* P;
  const void* P2;
  int64_t ldp, p_seg, p_row_seg;
  const void* Q;
  const void* Q2;
  int64_t ldq, q_row_seg;
  void* C;
  void* C2;
  int64_t ldc, c_seg, c_row_seg;
  const void* S1;
  const void* S2;
  const void* plan;        // BG_DH / BG_DX: plan buffer (header + entries)
  int64_t max_entries;     // grid of a plan-driven launch
  const int32_t* seg;      // BG_DW: [G+1] row offsets or null (dense_rows each)
  int32_t* order;          // BG_DW with seg: [G + 8] scratch: the longest-first segment
                           // order, then the 8 tile counters of the persistent launch
  int64_t dense_rows;
  const void* zero;        // BG_DW: >= 64 zero bf16 elements (16-byte aligned)
  int K, N, M, G;
  float* part;             // BG_DX whose plan has a tail split: the tail entries'
                           // fp32 partial tiles [kTailParts][256][256]
};
// 2 when a routed dX pass of this shape (K_all = both operand pairs) splits
// the tiles of its partial last round over K (the plan kernel decides from
// the real tile count), else 1.
int bwd_dx_split(int64_t rows, int G, int N, int K_all);
int bwd_tile_rows();
int bwd_tile_cols();
int64_t bwd_dw_blocks(int G, int M, int N);
hipError_t launch_bwd_gemm(const BwdGemm& b, hipStream_t s);

struct GateBwdArgs {
  const uint16_t* dy;       // [T, d]
  const uint16_t* eout;     // [T*k, d] expert outputs (bf16)
  const int32_t* slot_pos;  // [T*k]
  const int32_t* topk_idx;  // [T*k]
  const float* gate;        // [T*k]
  const float* logits;      // [T, E]
  const int32_t* counts;    // [E] (balance loss)
  float aux_scale;          // alpha E / T^2, 0 = no balance loss
  uint16_t* d_out;          // [T*k, d] dO on the permuted rows
  float* d_gate;            // [T, k] or null
  float* d_logits;          // [T, E]
  int64_t T;
  int d, k, E, gating;
};
hipError_t launch_gate_bwd(const GateBwdArgs& a, hipStream_t s);

struct DxArgs {
  const uint16_t* dxp;      // [T*k, d] per permuted row
  const uint16_t* dxs;      // [S, T, d] shared experts (S may be 0)
  const int32_t* slot_pos;
  const int32_t* topk_idx;
  const float* d_logits;    // [T, E]
  const uint16_t* w_router; // [E, d]
  uint16_t* dx;             // [T, d]
  int64_t T;
  int d, k, E, S;
  int sparse_ds;            // ds is zero outside the selected experts
};
hipError_t launch_dx(const DxArgs& a, hipStream_t s);

struct WrArgs {
  const float* d_logits;    // [T, E]
  const uint16_t* x;        // [T, d]
  float* dw_router;         // [E, d]
  float* partial;           // workspace, wr_ws_bytes()
  int64_t T;
  int E, d;
  int64_t chunk;            // set by the launcher
};
size_t wr_ws_bytes(int64_t T, int E, int d);
hipError_t launch_router_bwd(const WrArgs& a, hipStream_t s);
hipError_t launch_zero(void* p, size_t bytes, hipStream_t s);

}  // namespace moe
