// Kernel argument blocks and host-side launchers of libmoe (internal).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "noise.h"

namespace moe {

// ----------------------------------------------------------------- gate ----
struct GateFlatArgs {
  const void* x;
  const void* w_gate;   // [E][d]
  const void* w_noise;  // [E][d] or null
  const float* bias;    // [E] or null
  NoiseSrc noise;       // [T][E] tensor or generator; off: noise-free
  int64_t T;
  int d, E, k;
  int32_t* idx;   // [T][k]
  float* gate;    // [T][k]
  float* thr;     // [T][2] or null
  float* part;    // [ceil(T/32)][E] smooth-load partials (noisy, E <= 256) or null
  uint32_t* bits; // [ceil(T/32)][E] routing masks of the tile's tokens, or null
  float* imp_part = nullptr;  // [ceil(T/32)][E] gate sums of the tile's tokens (E <= 256) or null
  const void* w_pack = nullptr;  // packed tables (bf16, launch_pack_gate) or null
  int pack_nt = 0;               // tables in the packed form (1, or 2 with noise)
};
hipError_t launch_gate_flat(const GateFlatArgs& a, bool bf16, hipStream_t s);
// Packed gate tables: groups ng of eg experts (flat gate: ng = 1, eg = E),
// nt tables (w_gate, then w_noise when nt == 2), bf16, d % 64 == 0.
bool gate_pack_supported(bool bf16, int d);
size_t gate_packed_bytes(int ng, int eg, int d, int nt);
hipError_t launch_pack_gate(const void* w_gate, const void* w_noise, int ng, int eg, int d, int nt,
                            void* out, hipStream_t s);
constexpr int GATE_FUSED_LOAD_MAX_E = 256;
bool gate_fuses_load(int E);

struct GateGroupArgs {
  const void* x;
  const void* w_gate;   // [E][d], group g = rows g*Eg ..
  const void* w_noise;  // [E][d] or null
  NoiseSrc noise;       // [T][G][Eg] tensor or generator; off: noise-free
  int d, G, Eg, kg, kpg;
  const int32_t* perm_g;     // group routing of the primary selection
  const int32_t* offsets_g;  // [G+1]
  const int32_t* tiles_g;    // [G+1], tile_rows-row tiles per group (exclusive scan)
  int tile_rows = 32;        // 32 or 64
  const float* gate_p;       // [T][kg] primary gates
  int32_t* idx;              // [T][kg*kpg] final experts
  float* gate;               // [T][kg*kpg] final gates
  const void* w_pack = nullptr;  // packed secondary tables (G groups of Eg) or null
  int pack_nt = 0;
};
hipError_t launch_gate_group(const GateGroupArgs& a, int grid, bool bf16, hipStream_t s);
// Row tile of the secondary gate for `rows` (token, kept group) pairs over G
// groups: 64 for bf16 layers whose input tile fits LDS once the groups
// average 64 rows, else 32.  The group routing's tile map takes the same.
int gate_group_tile_rows(bool bf16, int d, int64_t rows, int G);

struct LoadArgs {
  const void* x;
  const void* w_gate;
  const void* w_noise;
  const float* bias;
  const int32_t* idx;  // [T][k]
  const float* thr;    // [T][2]
  int64_t T;
  int d, E, k;
  float* part;         // [ceil(T/32)][E]
  const void* w_pack = nullptr;  // packed tables (nt = 2) or null
};
int load_partial_blocks(int64_t T);
hipError_t launch_load_partial(const LoadArgs& a, bool bf16, hipStream_t s);

// ---------------------------------------------------------------- route ----
constexpr int ROUTE_BLOCK_TOKENS = 32;
struct RouteArgs {
  const int32_t* idx;  // [T][k]
  int64_t T;
  int k, E;
  int NB;              // ceil(T / 32)
  uint32_t* bits;      // [NB][E] workspace: bit i = token 32b+i kept e
  int32_t* base;       // [NB][E] workspace
  int have_bits;       // bits already written (by the flat gate)
  int32_t* counts;     // [E]
  int32_t* offsets;    // [E+1]
  int32_t* perm;       // [A]
  int32_t* inv;        // [A]
  int tile_rows;       // > 0: also build the expert tile map (tiles, desc)
  int32_t* tiles;      // [E+1]
  int32_t* desc;       // [tiles][3] or null
  // Balance statistics from per-block partials, reduced alongside the counts
  // (importance null: skipped).  load_part null: load = counts.
  const float* imp_part = nullptr;   // [NB][E]
  const float* load_part = nullptr;  // [NB][E] or null
  float* importance = nullptr;       // [E]
  float* load = nullptr;             // [E]
  float* bal_out = nullptr;          // [3]: CV^2(importance), CV^2(load), weighted sum
  float w_imp = 0.f, w_load = 0.f;
  // > 0: an expert keeps its first `capacity` assignments (token order); the
  // rest get inv = -1 and no position; counts / offsets count kept rows;
  // perm past offsets[E] holds 0.  The statistics above stay pre-drop.
  int capacity = 0;
};
hipError_t launch_route(const RouteArgs& a, hipStream_t s);
// Rows of a keep mask (bits [NB][E], one bit per token): counts per expert
// (capped at a.capacity when > 0), offsets, and perm[p] = the token at row
// p, tokens ascending inside each expert; perm[offsets[E] .. perm_len) = 0.
hipError_t launch_mask_route(const RouteArgs& a, int64_t perm_len, hipStream_t s);
hipError_t launch_fill_i32(int32_t* p, int n, int v, hipStream_t s);

// x_sorted[p] = x[perm[p] / k] for p < A (elem_bytes per element, d per row)
hipError_t launch_gather_rows(const void* x, const int32_t* perm, int k, int64_t A, int d,
                              int elem_bytes, void* out, hipStream_t s);

// tiles[e] = sum_{e' < e} ceil(count_{e'} / rows), tiles[E] = total; with
// desc != null also desc[q] = {expert, first position, rows} for every tile,
// an expert's 32-row blocks spread evenly over its tiles
hipError_t launch_tile_map(const int32_t* offsets, int E, int rows, int32_t* tiles,
                           int32_t* desc, hipStream_t s);

// --------------------------------------------------------------- experts ---
struct FfnArgs {
  const void* x;          // rows source
  const int32_t* perm;    // null: row p is x[p]; else x[perm[p] / k]
  int k;
  const int32_t* offsets; // [E+1]
  const int32_t* tiles;   // [E+1] tile map for the kernel's row tile (grouped
                          // GEMM paths; the fused path finds its tiles itself)
  int E, d, h;
  const void* w1;         // [E][h][d]
  const void* w3;         // [E][h][d] or null
  const void* w2;         // [E][d][h]
  void* hid;              // [A][h] workspace (unfused paths)
  void* y_sorted;         // [A][d]
  int64_t A;
  const void* wpacked;    // packed expert tables (fused path) or null
};
// rows per tile of the expert stage's tile map for A routed rows over E
// experts; 0 when the path needs no tile map (the fused path)
int ffn_tile_rows(bool bf16, int d, int h, int swiglu, int64_t A, int E);
// fused ReLU path (hidden layer kept on chip), d_model 512
bool fused_ffn_supported(int d, int h, int swiglu);
hipError_t launch_fused_ffn(const FfnArgs& a, hipStream_t s);
size_t fused_packed_bytes(int E, int d, int h);
hipError_t launch_pack_experts(const void* w1, const void* w2, int E, int d, int h, void* out,
                               hipStream_t s);
hipError_t launch_expert_ffn(const FfnArgs& a, bool bf16, int swiglu, hipStream_t s);

// The backward's hidden layer on the large-tile GEMM (bf16 layers whose
// experts average at least bw_hidden_big_rows() rows): recomputes the hidden
// activations and turns dHid into the pre-activation gradients.
struct BwHiddenArgs {
  const void* xs;          // [A][d] routed rows of x, in expert order
  const int32_t* offsets;  // [E+1]
  const int32_t* tiles;    // [E+1] tile map of bw_hidden_big_rows() rows
  int E, d, h;
  int64_t A;
  const void* w1;          // [E][h][d]
  const void* w3;          // [E][h][d] (SwiGLU) or null
  void* hid;               // [A][h] out: relu(a), or silu(a) b
  void* d1;                // [A][h] in: dHid = dY W2; out: dP (ReLU) or dA (SwiGLU)
  void* d3;                // [A][h] out: dB (SwiGLU) or null
};
// The ReLU hidden layer's recompute and gradient at d_model 512 on tiles of
// at most 96 rows of one expert (found by each workgroup
// from the offsets), the tables streamed once per tile: hid = relu(xs W1^T) and
// dp = (dys W2) * [xs W1^T > 0], both [A][h] bf16, where the kernel gathers
// xs and dys itself (and writes them out).
struct BwHidFusedArgs {
  const void* x;           // [T][512]
  const void* dy;          // [T][512] output gradients
  const int32_t* perm;     // [A] routing: position p holds assignment perm[p]
  const float* gate;       // [A] the assignments' gates
  int k;
  void* xs;                // [A][512] out: routed rows of x, in expert order
  void* dys;               // [A][512] out: gate-scaled output gradients, same order
  const int32_t* offsets;  // [E+1] routing offsets
  int E, h;
  const void* w1;          // [E][h][512]
  const void* w2;          // [E][512][h]
  const void* wp;          // the forward's packed tables (W1 read from them) or null
  void* hid;               // [A][h] out
  void* dp;                // [A][h] out
};
// dxs = dp W1 ([A][512] bf16) for the same layers, on the same tiles
struct BwDxFusedArgs {
  const void* dp;          // [A][h] bf16
  const int32_t* offsets;  // [E+1] routing offsets
  int E, h;
  const void* w1;          // [E][h][512]
  void* dxs;               // [A][512] out
};
hipError_t launch_bw_dx_fused(const BwDxFusedArgs& a, int64_t A, hipStream_t s);
bool bw_hidden_fused_supported(bool bf16, int d, int h, bool swiglu);
hipError_t launch_bw_hidden_fused(const BwHidFusedArgs& a, int64_t A, hipStream_t s);
bool bw_hidden_big_tiles(bool bf16, int64_t A, int E);
int bw_hidden_big_rows();
hipError_t launch_bw_hidden_big(const BwHiddenArgs& a, bool swiglu, hipStream_t s);
// c[p] = a[p] b_e (+ a2[p] b2_e) for the routed rows p of expert e, on the
// same large tiles; a, a2 [A][K] bf16 in expert order, b, b2 [E][K][N] bf16,
// c [A][N] bf16; N % 8 == 0, K % 64 == 0
struct BwBigProduct {
  const void* a;
  const void* a2;          // or null
  const void* b;
  const void* b2;          // or null
  int64_t A;
  int E, N, K;
  const int32_t* offsets;  // [E+1]
  const int32_t* tiles;    // [E+1] tile map of bw_hidden_big_rows() rows
  void* c;
};
hipError_t launch_bw_big_product(const BwBigProduct& p, hipStream_t s);
// c_e [M][N] = sum over the positions p of expert e of a[p][m] b[p][n], on
// the same large tiles; a [A][M], b [A][N] bf16 in expert order, c [E][M][N]
// bf16 (zero for an expert without rows); zero: max(M, N) bf16 zeros;
// M, N % 8 == 0
struct BwBigWgrad {
  const void* a;
  const void* b;
  int E, M, N;
  const int32_t* offsets;  // [E+1]
  const void* zero;
  void* c;
};
hipError_t launch_bw_big_wgrad(const BwBigWgrad& p, hipStream_t s);

// -------------------------------------------------------- combine / stats --
hipError_t launch_combine(const void* y_sorted, const int32_t* inv, const float* gate, int64_t T,
                          int k, int d, bool bf16, void* y, hipStream_t s);
// importance[e], load[e] (= sum_b part[b][e], or the row count when part is
// null), then the CV^2 / loss triple.
struct BalanceArgs {
  const int32_t* perm;     // expert-sorted assignments (token t, slot s) -> t*k + s
  const int32_t* offsets;  // [E+1]
  const float* gate;       // [T][k]
  const float* part;       // [blocks][E] or null
  int blocks, E, k;        // blocks = ceil(T / 32)
  float w_imp, w_load;
  float* importance;
  float* load;
  float* out;         // [3]
};
hipError_t launch_balance(const BalanceArgs& a, hipStream_t s);
// CV^2 of importance and load (fp64, fixed order) and their weighted sum
hipError_t launch_cv2(const float* importance, const float* load, int E, float w_imp,
                      float w_load, float* out, hipStream_t s);

// ------------------------------------------- per-batch equal-size mask ---
// In place of KeepTopK: expert e keeps the m tokens of the batch with the
// largest noisy scores (batch mask), or every token whose score reaches
// theta[e], at most m of them in token order (threshold mask).
struct MaskArgs {
  const void* x;
  const void* w_gate;   // [E][d]
  const void* w_noise;  // [E][d] or null
  const float* bias;    // [E] or null
  NoiseSrc noise;
  const void* w_pack = nullptr;  // packed gate tables or null
  int pack_nt = 1;
  int64_t T;
  int d, E;
  int NB;               // ceil(T / 32)
  int64_t Tp;           // row stride of Ht: 32 * NB
  int m;                // batch mask: rows per expert; threshold mask: the cap
  const float* theta;   // [E] threshold mask, or null (batch mask)
  float* Ht;            // [E][Tp] scores, expert-major
  uint32_t* bits;       // [NB][E] keep masks: bit i = token 32b+i kept by e
  const int32_t* base;  // [NB][E] kept tokens of e in blocks before b (colscan)
  const int32_t* offsets;  // [E+1] rows of each expert
  float2* tokstat;      // [T] max kept score, 1 / sum of exp over the kept experts
  int32_t* nslot;       // [T] kept pairs of the token that have a row
  int32_t* tok_off;     // [T+1]
  int32_t* slot_e;      // [rows] expert of each slot, ascending within a token
  float* slot_g;        // [rows] its gate
  int32_t* slot_pos;    // [rows] its row
  float* importance;    // [E] or null
  float* load;          // [E]
};
// scores (and, threshold mask, the keep masks)
hipError_t launch_mask_scores(const MaskArgs& a, bool bf16, bool noisy, hipStream_t s);
// batch mask: each expert's m best tokens -> keep masks
hipError_t launch_mask_select(const MaskArgs& a, hipStream_t s);
// per token: softmax statistics and slot counts; the slot offsets; the slots
hipError_t launch_mask_tokens(const MaskArgs& a, hipStream_t s);
// importance (gates recomputed from the token statistics) and hard load
hipError_t launch_mask_balance(const MaskArgs& a, hipStream_t s);
// y[t] = sum over the token's slots (ascending) of gate * y_sorted[row]
hipError_t launch_combine_csr(const void* y_sorted, const int32_t* tok_off,
                              const int32_t* slot_pos, const float* slot_g, int64_t T, int d,
                              bool bf16, void* y, hipStream_t s);

// -------------------------------------------------------------- backward ---
hipError_t launch_bw_cv2_grad(const float* imp, const float* load, int E, float wi, float wl,
                              float* dimp, float* dload, hipStream_t s);

struct BwGateOutArgs {
  const void* y_sorted;  // [A][d]
  const int32_t* inv;    // [A]
  const int32_t* idx;    // [T][k]
  const float* gate;     // [T][k]
  const void* dy;        // [T][d]
  const float* dimp;     // [E] or null
  int64_t T;
  int k, d;
  float* dhk;            // [T][k] gradient of the kept noisy scores
};
hipError_t launch_bw_gate_out(const BwGateOutArgs& a, bool bf16, hipStream_t s);

struct BwGateArgs {
  const void* x;
  const void* w_gate;
  const void* w_noise;   // null: noise-free gate
  const float* bias;
  NoiseSrc noise;        // [T][E] tensor or generator (noisy)
  const void* w_pack = nullptr;
  int pack_nt = 0;
  const int32_t* idx;    // [T][k]
  const float* thr;      // [T][2] (smooth load) or null
  const float* dload;    // [E] load-loss gradient or null (no smooth-load term)
  const float* dhk;      // [T][k]
  int64_t T;
  int d, E, k;
  int32_t* rinfo;        // [T][4]: expert ranked k, k+1 (-1: none), their score gradients
  float* dclean;         // [T][E] fp32, or null when written as bf16 halves below
  float* draw;           // [T][E] (noisy)
  // bf16 layers: the score gradients as bf16 hi and lo halves (hi = the
  // rounded value, lo = the rounded remainder), [T][E] each, the operands the
  // products take; null: fp32 dclean / draw above
  bf16_t* dclean_hi = nullptr;
  bf16_t* dclean_lo = nullptr;
  bf16_t* draw_hi = nullptr;
  bf16_t* draw_lo = nullptr;
  float* dbias_part;     // [ceil(T/32)][E]
  // bf16 layers with E <= 256: the gate's share of dx, dclean W_gate +
  // draw W_noise, is formed in the same kernel from the tile's score
  // gradients (bf16 hi + lo halves) and the tables transposed to
  // [d][ceil(E/16)*16] (zero past E); null: a separate product forms it
  const bf16_t* wgt = nullptr;
  const bf16_t* wnt = nullptr;
  int e16 = 0;
  float* dxg = nullptr;  // [T][d]
};
// the largest expert count for which the gate-gradient kernel forms dx_gate
int bw_fused_dxg_max_experts();
// out[c][e] = in[e][c] for e < E, 0 for E <= e < e16 (in [E][d], out [d][e16])
hipError_t launch_bw_transpose_table(const void* in, int E, int d, int e16, void* out,
                                     hipStream_t s);
// The hierarchy's gate gradients, one wave per token.  A kept gate is the
// product gp[a] * gs[a, b] of the two levels' softmax weights; with V_a the
// sum over group a's slots of gs * dgate, the secondary score gradient of
// slot s is gate_s (dgate_s - V_a) and the primary score gradient of kept
// group a is gp_a (V_a - sum over kept groups of gp V).  Each then passes
// through its noisy score
// (d raw = dH * eps * sigmoid(raw)) to dx and to per-slot / per-group
// coefficients for the table gradients.
struct BwHierGateArgs {
  const void* y_sorted;  // [A][d]
  const int32_t* inv;    // [A]
  const int32_t* idx;    // [T][k], group-major (ascending expert index)
  const float* gate;     // [T][k]
  const void* dy;        // [T][d]
  const float* dimp;     // [E] or null
  const void* x;         // [T][d]
  const void* w_gate;    // [E][d]
  const void* w_noise;   // [E][d], null when noise-free
  const void* w_gate_p;  // [G][d]
  const void* w_noise_p; // [G][d], null when noise-free
  NoiseSrc noise;        // secondary: element j of group g of token t
  NoiseSrc noise_p;      // primary: element g of token t
  int64_t T;
  int k, d, G, Eg, kpg;
  float* dxg;            // [T][d] the gate's share of dx
  float* cs;             // [T*k] secondary clean-score gradient per slot
  float* ns;             // [T*k] secondary raw-score gradient per slot (null: noise-free)
  float* dcp;            // [T][G] primary clean-score gradient (0 outside kept groups)
  float* drp;            // [T][G] primary raw-score gradient (null: noise-free)
};
hipError_t launch_bw_hier_gate(const BwHierGateArgs& a, bool bf16, hipStream_t s);

// out0[e] = sum over the rows p of expert e (offsets / perm, in order) of
// c0[perm[p]] * x[perm[p] / k], likewise out1 with c1 (nullable); experts
// with no rows get zeros.
struct BwRowSumArgs {
  const void* x;           // [T][d]
  const int32_t* perm;     // [A]
  const int32_t* offsets;  // [E+1]
  const float* c0;         // [T*k]
  const float* c1;         // [T*k] or null
  int k, E, d;
  void* out0;              // [E][d]
  void* out1;              // [E][d] or null
};
hipError_t launch_bw_expert_rowsum(const BwRowSumArgs& a, bool bf16, hipStream_t s);

size_t bw_gate_lds_bytes(bool bf16, int d, int E);
hipError_t launch_bw_gate(const BwGateArgs& a, bool bf16, hipStream_t s);
hipError_t launch_bw_sum_rows(const float* part, int64_t nrow, int64_t ncol, float* out,
                              hipStream_t s);
hipError_t launch_bw_sum_chunks(const float* part, int nchunk, int64_t n, bool bf16, void* out,
                                hipStream_t s);
// dx = dxg + the routed rows' dxs (in the layer dtype), skipping dropped slots
hipError_t launch_bw_assemble_dx(const float* dxg, const void* dxs, const int32_t* inv, int64_t T,
                                 int k, int d, bool bf16, void* dx, hipStream_t s);

// Operand of a backward product: element (r, k) of an R x K matrix, for
// problem (expert) e at p + e*estride + (kind KB/KF: r*ld + k; TB/TF:
// k*ld + r); B = bf16, F = fp32.  Kinds KB and TB need K % 8 == 0 (KB) and
// R % 4 == 0 (TB) and ld % 8 == 0.
// TD: a TB operand the launcher loads straight into LDS (set by launch_bw_gemm)
enum { BW_KB = 0, BW_TB = 1, BW_KF = 2, BW_TF = 3, BW_TD = 4 };
struct BwOp {
  const void* p = nullptr;
  int64_t estride = 0;
  int64_t ld = 0;
  int kind = BW_KB;
  int lo = 0;                   // bf16 products: the residual v - bf16(v) of each value
};
enum { BW_POS = 0, BW_WGT = 1, BW_PLAIN = 2 };
enum { BW_EPI_NONE = 0, BW_EPI_RELU = 1, BW_EPI_SWIGLU = 2 };
struct BwGemm {
  int mode = BW_PLAIN;
  int epi = BW_EPI_NONE;
  // plain: C = sum over the npair pairs of a[i] b[i]^T (same kinds for every
  // pair: a second table, or the low halves of fp32 operands); hidden:
  // (a[0], b[0]) = (X, W1), (a[1], b[1]) = (dY, W2^T), (a[0], b[2]) = (X, W3)
  BwOp a[4], b[4];
  int npair = 1;
  int64_t M = 0, N = 0, K = 0;
  int64_t kchunk = 0;           // PLAIN: K per chunk (grid covers the chunks)
  const int32_t* offsets = nullptr;  // [E+1]
  const int32_t* tiles = nullptr;    // POS: [E+1] row tiles of pos_rows rows
  int pos_rows = 128;                // POS: rows per tile, bw_pos_tile_rows()
  const void* zero = nullptr;        // WGT, bf16: >= 128 zero elements (or null)
  int E = 0;
  void* C = nullptr;            // plain: output; hidden: Hid [A][N]
  void* C2 = nullptr;           // hidden: dP (ReLU) or dA (SwiGLU)
  void* C3 = nullptr;           // SwiGLU: dB
  int c_f32 = 1;
  int64_t ldc = 0, c_estride = 0, c_chunk = 0;
  int nrow = 0, ncol = 0;       // set by the launcher
};
// out[p] = src[perm[p] / k] (times scale[perm[p]]), d % 8 == 0 (bf16) or % 4 (fp32)
hipError_t launch_bw_gather_rows(const void* src, const int32_t* perm, int k, const float* scale,
                                 int64_t A, int d, bool bf16, void* out, hipStream_t s);
// Rows per tile of the row-position products (the hidden recompute and dX):
// 32 when a bf16 layer's experts average at most 32 rows, else 128.
int bw_pos_tile_rows(bool bf16, int64_t A, int E);
hipError_t launch_bw_gemm(BwGemm g, bool bf16, int64_t grid, hipStream_t s);

}  // namespace moe

namespace moe {
// eps [T][E] (flat) or eps [T][G][Eg] and eps_p [T][G] (hierarchy, G > 0)
// drawn from the generator; either may be null
hipError_t launch_draw_noise(int64_t T, int E, int G, uint64_t seed, float* eps, float* eps_p,
                             hipStream_t s);
}  // namespace moe
